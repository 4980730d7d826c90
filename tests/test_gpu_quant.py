"""GPU parity of attn_quantize_qk (K mean, smoothing, per-block INT8 Q/K) against
the CPU oracle: every output is bit-exact (the reading of the SageAttention
article's 技术方案 section fixes a unique result; see include/attn.h)."""
import numpy as np
import pytest
import torch

import bit_quantized_exact_amd as A
from bit_quantized_exact_amd.inputs import WORKLOADS, make_qkv
from oracle import oracle as O

from _util import case, dev, host, small_workload

pytestmark = pytest.mark.gpu

SMALL = [
    (1, 2, 2, 1, 64), (1, 2, 1, 7, 128), (1, 2, 2, 16, 64), (1, 4, 2, 17, 128),
    (2, 2, 2, 63, 64), (1, 2, 2, 64, 128), (1, 3, 3, 65, 64), (1, 4, 1, 127, 128),
    (1, 2, 2, 128, 64), (2, 4, 2, 129, 128), (1, 2, 2, 255, 64), (1, 2, 1, 257, 128),
    (1, 8, 2, 1000, 128), (3, 2, 2, 513, 64),
    # 32 chunk sums (the K quantiser adds them itself) and 33 (the mean kernel runs)
    (1, 2, 1, 8192, 64), (1, 2, 2, 8193, 128),
]


def _compare(w, q, k):
    case(f"quantize {w.name} B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} S={w.seq} D={w.head_dim}")
    got = A.quantize_qk(dev(q), dev(k))
    torch.cuda.synchronize()
    ref = O.quantize_qk(q, k)
    for key in ("k_mean", "q_scale", "k_scale", "q_i8", "k_i8"):
        g = host(got[key])
        r = ref[key]
        assert g.shape == r.shape, key
        if not np.array_equal(g.view(np.uint8) if g.dtype == np.int8 else g.view(np.uint32),
                              r.view(np.uint8) if r.dtype == np.int8 else r.view(np.uint32)):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{key}: {len(bad)} mismatches, first at {bad[:3].tolist()}: "
                                 f"{g[tuple(bad[0])]} vs {r[tuple(bad[0])]}")


@pytest.mark.parametrize("B,Hq,Hkv,S,D", SMALL)
def test_quantize_bitexact_small(B, Hq, Hkv, S, D):
    w = small_workload(B, Hq, Hkv, S, D, False, seed=S * 13 + D)
    q, k, _ = make_qkv(w)
    _compare(w, q, k)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_quantize_bitexact_workloads(name):
    w = WORKLOADS[name]
    q, k, _ = make_qkv(w)
    _compare(w, q, k)


def test_quantize_special_blocks():
    """Constant K (smoothed K is exactly zero: delta 0, q 0), an all-zero Q
    block, and exact ties of x*127/a."""
    w = small_workload(1, 2, 2, 200, 64, False, seed=5)
    q, k, _ = make_qkv(w)
    k[0, 0] = np.float16(3.5)             # every token equal -> ks = 0
    q[0, 1, 128:200] = 0                   # the second (partial) Q block is zero
    # a block whose absmax is 127 * 2^-3: x*r is exact and multiples of 0.5 * 2^-3 tie
    ints = (np.arange(128 * 64).reshape(128, 64) % 255 - 127).astype(np.float64)
    blk = ints * 0.125
    odd = np.zeros_like(blk, dtype=bool)
    odd[1::2] = np.abs(ints[1::2]) < 126
    blk[odd] += 0.0625                     # x * 8 = k + 1/2 exactly
    assert np.abs(blk).max() == 127 * 0.125
    q[0, 0, :128] = blk.astype(np.float16)
    _compare(w, q, k)
    ref = O.quantize_qk(q, k)
    assert (ref["k_scale"][0, 0] == 0).all() and not ref["k_i8"][0, 0].any()
    assert ref["q_scale"][0, 1, 1] == 0


def test_quantize_ignores_workspace_contents_and_is_deterministic():
    w = small_workload(1, 4, 2, 700, 128, False, seed=9)
    q, k, _ = make_qkv(w)
    qd, kd = dev(q), dev(k)
    case("quantize workspace garbage / determinism")
    a = A.quantize_qk(qd, kd)
    ws = a["workspace"]
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=ws.device))
    b = A.quantize_qk(qd, kd, workspace=ws)
    torch.cuda.synchronize()
    for key in ("k_mean", "q_scale", "k_scale", "q_i8", "k_i8"):
        assert torch.equal(a[key], b[key]), key


def test_quantize_k_mean_exact_under_cancellation():
    """Channel sums that no fp32 summation order gets right: +-65504 pairs that
    cancel around fp16 subnormals (2^-24), a channel of 65504 everywhere, and
    a channel of one subnormal per token; the mean must match the oracle's
    exact sum bit for bit across several 256-token sum chunks and a ragged
    tail."""
    w = small_workload(1, 2, 2, 1000, 64, False, seed=11)
    q, k, _ = make_qkv(w)
    S = w.seq
    tiny = np.float16(2.0 ** -24)
    col = np.where(np.arange(S) % 2 == 0, np.float16(65504.0), np.float16(-65504.0))
    col[::7] = tiny                              # breaks the pairing: the sum is dominated by +-65504
    k[0, 0, :, 0] = col
    k[0, 0, :, 1] = np.float16(65504.0)
    k[0, 0, :, 2] = tiny
    k[0, 1, :, 3] = -tiny
    k[0, 1, ::3, 3] = np.float16(-65504.0)
    _compare(w, q, k)
    ref = O.quantize_qk(q, k)
    exact = k[0, 0, :, 2].astype(np.float64).sum() / S
    assert ref["k_mean"][0, 0, 2] == np.float32(exact)


def test_quantize_bitexact_at_the_maximum_sequence():
    """ATTN_MAX_SEQ = 2^22 tokens, the longest sequence the ABI accepts and the
    length up to which the fixed-point channel sums are exact: every output
    bit-exact against the oracle (one q-head on one kv-head, head_dim 128)."""
    w = small_workload(1, 1, 1, 1 << 22, 128, False, seed=71)
    q, k, _ = make_qkv(w)
    _compare(w, q, k)


def test_k_mean_exact_at_the_maximum_sequence_extremes():
    """At 2^22 tokens, channels whose exact means are known without the oracle
    (which refuses sums this large): constant +65504, constant -65504, the
    smallest subnormal 2^-24 everywhere, and one 65504 among 2^-24s (a sum
    that loses every small term in any fp32 order).  The mean is the exact
    sum, rounded once to fp64, divided by S and rounded to fp32."""
    S = 1 << 22
    tiny = 2.0 ** -24
    k = np.zeros((1, 1, S, 64), dtype=np.float16)
    k[0, 0, :, 0] = np.float16(65504.0)
    k[0, 0, :, 1] = np.float16(-65504.0)
    k[0, 0, :, 2] = np.float16(tiny)
    k[0, 0, :, 3] = np.float16(tiny)
    k[0, 0, 0, 3] = np.float16(65504.0)
    case("quantize_k 2^22 tokens, extreme channel sums")
    got = A.quantize_k(dev(k))
    torch.cuda.synchronize()
    mean = host(got["k_mean"])[0, 0]
    want = np.zeros(64, dtype=np.float32)
    want[0], want[1], want[2] = 65504.0, -65504.0, np.float32(tiny)
    want[3] = np.float32((65504.0 + (S - 1) * tiny) / S)
    assert want[3] != np.float32(65504.0 / S)          # the small terms matter
    np.testing.assert_array_equal(mean.view(np.uint32), want.view(np.uint32))

