"""GPU parity of the KV-cache (decode) kernels against the CPU oracle.

"注意力即一切：从 MHA 到 GQA" §3.4: the current token's queries attend over
the cached keys and values; the queries are the last Sq positions (causal
mask aligned bottom-right).

* attn_decode_int8: the in-kernel Q block scales bit-exact against the
  oracle's quantiser; O max-abs <= 2e-3 and lse within 1e-4 against the
  oracle's quantised KV model (same INT8 codes); cosine >= 0.999 and relative
  L1 <= 0.02 against exact attention.
* attn_decode_fp16: max-abs <= 2e-3 against exact fp64 attention.
* Shapes cover Sq = 1..32, caches of 1 to 8192 keys (tails of every tile
  class), GQA/MQA/MHA, an explicit irregular head map, several query chunks
  per kv-head and the full-size decode workload; plus run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import bit_quantized_exact_amd as A
from bit_quantized_exact_amd.inputs import DECODE_WORKLOADS, Workload, make_qkv
from oracle import oracle as O

from _util import FP16_MAX_ABS, INT8_COS_MIN, INT8_REL_L1_MAX, INT8_VS_MODEL_MAX_ABS, case, cos_rel_l1, dev, host

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, map
    (1, 4, 2, 1, 1, 128, True, None),
    (1, 4, 2, 1, 33, 64, True, None),
    (2, 8, 2, 3, 100, 128, True, None),
    (1, 16, 1, 5, 1000, 128, True, None),
    (1, 4, 4, 32, 64, 64, False, None),
    (2, 6, 3, 8, 2049, 64, True, None),
    (1, 5, 3, 7, 300, 128, True, [2, 0, 2, 1, 0]),
    (1, 40, 1, 32, 500, 64, True, None),
    (1, 32, 8, 16, 4096, 128, True, None),
    (2, 2, 2, 2, 2, 128, False, None),
    (1, 4, 3, 4, 260, 64, True, [0, 2, 2, 0]),   # kv-head 1 unused
]


def _w(c, seed):
    B, Hq, Hkv, Sq, Sk, D, causal, _ = c
    return Workload(f"dec_{B}x{Hq}x{Hkv}x{Sq}x{Sk}x{D}", B, Hq, Hkv, Sk, D, causal, 3.0, seed=seed, seq_q=Sq)


def _int8_check(w, q, k, v, kv_map=None):
    case(f"decode_int8 {w.name} causal={w.causal} map={kv_map}")
    kz = A.quantize_k(dev(k))
    qs = torch.empty((w.batch, w.heads_q), dtype=torch.float32, device="cuda")
    out, lse = A.decode_int8(dev(q), kz, dev(v), causal=w.causal, kv_head_map=kv_map, return_lse=True,
                             q_scale_out=qs)
    torch.cuda.synchronize()
    got, gl = host(out).astype(np.float64), host(lse).astype(np.float64)
    qi, qsc = O.quantize_q(q)
    assert np.array_equal(host(qs), qsc[..., 0]), "Q block scales differ"
    kc = O.quantize_k_cache(k)
    assert np.array_equal(host(kz["k_i8"]), kc["k_i8"]) and np.array_equal(host(kz["k_scale"]), kc["k_scale"])
    model, ml = O.quant_attention_kv(qi, qsc, kc, v, causal=w.causal, kv_map=kv_map, with_lse=True)
    err = np.abs(got - model).max()
    assert err <= INT8_VS_MODEL_MAX_ABS, f"max-abs vs quantised model {err}"
    assert np.abs(gl - ml).max() <= 1e-4
    exact = O.attention_kv(q, k, v, causal=w.causal, kv_map=kv_map)
    cos, rel = cos_rel_l1(got, exact)
    assert cos >= INT8_COS_MIN and rel <= INT8_REL_L1_MAX, (cos, rel)
    return out


def _fp16_check(w, q, k, v, kv_map=None):
    case(f"decode_fp16 {w.name} causal={w.causal} map={kv_map}")
    out, lse = A.decode_fp16(dev(q), dev(k), dev(v), causal=w.causal, kv_head_map=kv_map, return_lse=True)
    torch.cuda.synchronize()
    exact, el = O.attention_kv(q, k, v, causal=w.causal, kv_map=kv_map, with_lse=True)
    err = np.abs(host(out).astype(np.float64) - exact).max()
    assert err <= FP16_MAX_ABS, f"max-abs {err}"
    assert np.abs(host(lse).astype(np.float64) - el).max() <= 1e-3
    return out


@pytest.mark.parametrize("c", CASES, ids=lambda c: "x".join(map(str, c[:7])))
def test_decode_int8(c):
    w = _w(c, 21)
    q, k, v = make_qkv(w)
    _int8_check(w, q, k, v, kv_map=c[7])


@pytest.mark.parametrize("c", CASES, ids=lambda c: "x".join(map(str, c[:7])))
def test_decode_fp16(c):
    w = _w(c, 22)
    q, k, v = make_qkv(w)
    _fp16_check(w, q, k, v, kv_map=c[7])


def test_decode_workload_full_size():
    w = DECODE_WORKLOADS["decode_gqa"]
    q, k, v = make_qkv(w)
    _int8_check(w, q, k, v)
    _fp16_check(w, q, k, v)


def test_decode_is_deterministic():
    w = _w((2, 8, 2, 4, 3000, 128, True, None), 23)
    q, k, v = make_qkv(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    case("decode determinism")
    kz = A.quantize_k(kd)
    a = A.decode_int8(qd, kz, vd).clone()
    b = A.decode_int8(qd, kz, vd)
    c = A.decode_fp16(qd, kd, vd).clone()
    d = A.decode_fp16(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


def test_decode_rows_match_prefill_rows():
    """Bottom-right alignment on the GPU: the decode of the last Sq queries
    agrees with the last Sq rows of the square FP16 forward over the same
    sequence (both within the FP16 tolerance of exact attention)."""
    Sk, Sq = 700, 5
    w = Workload("dec_vs_prefill", 1, 4, 2, Sk, 64, True, 2.0, seed=24)
    q_full, k, v = make_qkv(w)
    case("decode vs prefill rows")
    dec = A.decode_fp16(dev(np.ascontiguousarray(q_full[:, :, Sk - Sq:])), dev(k), dev(v), causal=True)
    pre = A.fwd_fp16(dev(q_full), dev(k), dev(v), causal=True)
    torch.cuda.synchronize()
    diff = (dec.float() - pre[:, :, Sk - Sq:].float()).abs().max().item()
    assert diff <= 2 * FP16_MAX_ABS, diff


def test_decode_at_the_maximum_cache():
    """A cache of ATTN_MAX_SEQ = 2^22 keys (1 GiB each of K and V at head_dim
    128): 1024 key splits merged by the combine kernel; the cache quantisation
    bit-exact, both decode kernels against the oracle as above."""
    w = _w((1, 4, 1, 3, 1 << 22, 128, True, None), seed=977)
    q, k, v = make_qkv(w)
    _int8_check(w, q, k, v)
    _fp16_check(w, q, k, v)

