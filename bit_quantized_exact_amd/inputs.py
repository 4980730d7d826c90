"""Seeded synthetic attention inputs (no attention arithmetic lives here).

This module only draws random fp16 tensors.  It is shared by the HIP path's
tests and benchmark and by the CPU oracle's tests, and it computes nothing the
method computes: no mean, no quantisation, no score.

Workloads
---------
Each workload is a Q/K/V triple in ``[batch, heads, seq, head_dim]`` layout,
row-major, fp16.  The value recipe follows what the SageAttention article
(jiqizhixin reprint, "Challenges" section) reports about real models: the K
matrix carries strong *channel-wise* outliers, i.e. a bias per channel shared by
every token.  We model that as ``K = noise + offset[channel]`` with the offset
drawn once per (batch, kv-head, channel).  Q and V are plain N(0, 1).

Random streams: one ``numpy.random.default_rng([seed, t])`` per tensor, with
``t`` = 0 for Q, 1 for the K noise, 2 for V, 3 for the K offsets and 4 for the
choice of outlier channels, so every tensor is reproducible on its own.
"""
from __future__ import annotations

import dataclasses
import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_OFFSET, STREAM_OUTLIER = range(5)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seq: int
    head_dim: int
    causal: bool
    offset_std: float          # std of the per-channel K offset
    outlier_frac: float = 0.0  # fraction of channels whose offset is x10
    via_bf16: bool = False     # draw fp32, round to bf16, then to fp16
    seed: int = 0
    seq_q: int = 0             # queries per head when they differ from seq (KV-cache
                               # decode: the last seq_q positions of a seq-token cache)

    @property
    def n_q(self) -> int:
        return self.seq_q if self.seq_q else self.seq

    @property
    def q_shape(self):
        return (self.batch, self.heads_q, self.n_q, self.head_dim)

    @property
    def kv_shape(self):
        return (self.batch, self.heads_kv, self.seq, self.head_dim)

    def flops(self) -> float:
        """4*B*Hq*S^2*D, halved when causal (two contractions of 2*S*S*D each).
        With seq_q queries over a seq-token cache: 4*B*Hq*D per visible
        (query, key) pair, seq_q*seq pairs, or seq_q*(seq-seq_q) +
        seq_q*(seq_q+1)/2 when causal (bottom-right aligned)."""
        if self.seq_q:
            sq, sk = self.seq_q, self.seq
            pairs = sq * (sk - sq) + sq * (sq + 1) / 2 if self.causal else sq * sk
            return 4.0 * self.batch * self.heads_q * self.head_dim * pairs
        f = 4.0 * self.batch * self.heads_q * self.seq * self.seq * self.head_dim
        return f / 2 if self.causal else f

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five synthetic workloads: a tiny case, LLM prefill with GQA, a
# video-diffusion style MHA, long-context GQA and batched short MQA.
WORKLOADS = {
    "tiny_mha": Workload("tiny_mha", 1, 2, 2, 128, 64, False, 2.0, seed=0),
    "llm_prefill_gqa": Workload("llm_prefill_gqa", 1, 32, 8, 8192, 128, True, 4.0,
                                outlier_frac=0.01, seed=1),
    "video_mha": Workload("video_mha", 2, 24, 24, 16384, 64, False, 3.0,
                          via_bf16=True, seed=2),
    "long_gqa": Workload("long_gqa", 1, 32, 8, 32768, 128, True, 4.0, seed=3),
    "batched_mqa": Workload("batched_mqa", 64, 16, 1, 1024, 128, True, 2.0, seed=4),
}


# KV-cache decode: one new token per sequence (seq_q = 1) attending over an
# 8192-token cache, LLaMA-style 32 q-heads / 8 kv-heads, a batch of 16.
DECODE_WORKLOADS = {
    "decode_gqa": Workload("decode_gqa", 16, 32, 8, 8192, 128, True, 4.0, outlier_frac=0.01,
                           seed=5, seq_q=1),
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def _round_to_bf16(x32: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even), returned as float32."""
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _to_f16(x32: np.ndarray, via_bf16: bool) -> np.ndarray:
    if via_bf16:
        x32 = _round_to_bf16(x32)
    return x32.astype(np.float16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def k_offsets(w: Workload) -> np.ndarray:
    """Per (batch, kv-head, channel) K offsets, float32 [B, Hkv, 1, D]."""
    off = _normal(_rng(w.seed, STREAM_OFFSET), (w.batch, w.heads_kv, 1, w.head_dim))
    off *= np.float32(w.offset_std)
    if w.outlier_frac > 0:
        n_out = max(1, int(round(w.outlier_frac * w.head_dim)))
        pick = _rng(w.seed, STREAM_OUTLIER)
        for b in range(w.batch):
            for h in range(w.heads_kv):
                ch = pick.choice(w.head_dim, size=n_out, replace=False)
                off[b, h, 0, ch] *= np.float32(10.0)
    return off


def make_qkv(w: Workload):
    """Return (q, k, v) as contiguous float16 numpy arrays in [B, H, S, D]."""
    q = _to_f16(_normal(_rng(w.seed, STREAM_Q), w.q_shape), w.via_bf16)
    kn = _normal(_rng(w.seed, STREAM_K), w.kv_shape)
    kn += k_offsets(w)
    k = _to_f16(kn, w.via_bf16)
    del kn
    v = _to_f16(_normal(_rng(w.seed, STREAM_V), w.kv_shape), w.via_bf16)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)


def default_kv_map(heads_q: int, heads_kv: int) -> np.ndarray:
    """Contiguous grouping: q-head h reads kv-head h // (Hq / Hkv)."""
    g = heads_q // heads_kv
    return (np.arange(heads_q, dtype=np.int32) // g).astype(np.int32)


def sample_rows(seq: int, n_random: int, seed: int, block: int = 128) -> np.ndarray:
    """Sorted query-row sample: block edges, the middle, the last row, plus random rows."""
    fixed = {0, 1, block - 1, block, seq // 2, seq - 1}
    rows = {r for r in fixed if 0 <= r < seq}
    rng = np.random.default_rng([seed, 99])
    if n_random > 0:
        rows |= set(int(x) for x in rng.integers(0, seq, size=n_random))
    return np.array(sorted(rows), dtype=np.int32)
