"""GPU parity of the fused forward kernels against the CPU oracle.

* INT32 score tiles: bit-exact against the oracle's integer scores, as the
  INT8 forward kernels compute them -- attn_debug_qk_int32 runs the kernel of
  attn_fwd_int8 and attn_debug_qk_int32_fused_q that of attn_fwd_int8_fused_q
  (same copies into LDS, LDS layout, score MFMAs and work schedule), writing
  the INT32 tiles in place of the softmax; the fused dump's Q block scales
  are bit-exact too.
* FP16 path (attn_fwd_fp16): max-abs <= 2e-3 against fp64 exact attention.
* INT8 path (attn_fwd_int8): cosine >= 0.999 and relative L1 <= 0.02 against
  fp64 exact attention; max-abs <= 2e-3 against the oracle's quantised model
  (which separates kernel error from quantisation error).
* Invariants from the pages: a constant V gives that constant, causal row 0
  gives V_0, GQA/MQA share K/V per group; plus run-to-run determinism.

Small cases cover every tail class (S = 1..17, 63-65, 127-129, 1000), both
head dims, MHA/GQA/MQA and an explicit non-contiguous map; the workload
cases run the full-size launch and compare sampled rows."""
import numpy as np
import pytest
import torch

import bit_quantized_exact_amd as A
from bit_quantized_exact_amd.inputs import WORKLOADS, make_qkv, sample_rows
from oracle import oracle as O

from _util import (FP16_MAX_ABS, INT8_COS_MIN, INT8_REL_L1_MAX, INT8_VS_MODEL_MAX_ABS, case,
                   cos_rel_l1, dev, host, small_workload)

pytestmark = pytest.mark.gpu

TAILS = list(range(1, 18)) + [63, 64, 65, 127, 128, 129, 1000]


def _fp16_check(w, q, k, v, rows=None, kv_map=None):
    case(f"fwd_fp16 {w.name} S={w.seq} D={w.head_dim} causal={w.causal} map={kv_map}")
    out = A.fwd_fp16(dev(q), dev(k), dev(v), causal=w.causal, kv_head_map=kv_map)
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    if rows is not None:
        got = got[:, :, rows]
    ref = O.attention(q, k, v, causal=w.causal, kv_map=kv_map, rows=rows)
    err = np.abs(got - ref).max()
    assert err <= FP16_MAX_ABS, f"max-abs {err}"
    return err


def _int8_check(w, q, k, v, rows=None, kv_map=None):
    case(f"fwd_int8 {w.name} S={w.seq} D={w.head_dim} causal={w.causal} map={kv_map}")
    qz = A.quantize_qk(dev(q), dev(k))
    out = A.fwd_int8(qz, dev(v), causal=w.causal, kv_head_map=kv_map)
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    if rows is not None:
        got = got[:, :, rows]
    exact = O.attention(q, k, v, causal=w.causal, kv_map=kv_map, rows=rows)
    cos, rel = cos_rel_l1(got, exact)
    assert cos >= INT8_COS_MIN and rel <= INT8_REL_L1_MAX, (cos, rel)
    qz_h = {key: host(qz[key]) for key in ("q_i8", "q_scale", "k_i8", "k_scale")}
    model = O.quant_attention(qz_h, v, causal=w.causal, kv_map=kv_map, rows=rows)
    err = np.abs(got - model).max()
    assert err <= INT8_VS_MODEL_MAX_ABS, f"max-abs vs quantised model {err}"
    return cos, rel, err


# --------------------------------------------------------------------------
# integer score tiles: bit-exact
# --------------------------------------------------------------------------
def _dump_check(w, q, k, tiles, kv_map=None):
    """Both INT8 kernels' score tiles (INT8 Q from the oracle's quantiser, and
    fp16 Q quantised in the fused kernel) against the oracle's scores."""
    qz = O.quantize_qk(q, k)
    nqt = -(-w.seq // 128)
    qd, kd = dev(q), dev(qz["k_i8"])
    for lo, hi in tiles:
        hi = min(hi, nqt - 1)
        rows = np.arange(lo * 128, min((hi + 1) * 128, w.seq))
        ref = O.scores_i32(qz["q_i8"], qz["k_i8"], causal=w.causal, kv_map=kv_map, rows=rows,
                           fill=-(1 << 31))
        for fused in (False, True):
            case(f"debug_qk_int32{'_fused_q' if fused else ''} {w.name} S={w.seq} D={w.head_dim} "
                 f"causal={w.causal} tiles {lo}..{hi} map={kv_map}")
            if fused:
                qs = torch.full(qz["q_scale"].shape, -1.0, dtype=torch.float32, device="cuda")
                s = A.debug_qk_int32_fused_q(qd, kd, causal=w.causal, kv_head_map=kv_map, tile_lo=lo,
                                             tile_hi=hi, fill=-(1 << 31), q_scale_out=qs)
            else:
                s = A.debug_qk_int32(dev(qz["q_i8"]), kd, causal=w.causal, kv_head_map=kv_map,
                                     tile_lo=lo, tile_hi=hi, fill=-(1 << 31))
            torch.cuda.synchronize()
            got = host(s)
            g = got[:, :, :len(rows)]
            assert np.array_equal(g, ref), f"{np.count_nonzero(g != ref)} mismatching scores"
            # rows beyond S stay untouched
            assert (got[:, :, len(rows):] == -(1 << 31)).all()
            del s, got, g
            if fused:
                hq = host(qs)
                assert np.array_equal(hq[:, :, lo:hi + 1], qz["q_scale"][:, :, lo:hi + 1])
                untouched = np.ones(hq.shape[2], dtype=bool)
                untouched[lo:hi + 1] = False
                assert (hq[:, :, untouched] == -1.0).all()


@pytest.mark.parametrize("S", [1, 5, 16, 17, 64, 65, 127, 128, 129, 300])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_int32_scores_bitexact_small(S, D, causal):
    w = small_workload(1, 4, 2, S, D, causal, seed=S + D)
    q, k, _ = make_qkv(w)
    nqt = -(-S // 128)
    _dump_check(w, q, k, [(0, nqt - 1)])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_int32_scores_bitexact_workloads(name):
    w = WORKLOADS[name]
    q, k, _ = make_qkv(w)
    nqt = -(-w.seq // 128)
    # the first, a middle and the last query tile of every (batch, head)
    _dump_check(w, q, k, [(0, 0), (nqt // 2, nqt // 2), (nqt - 1, nqt - 1)])


def test_int32_scores_explicit_map():
    w = small_workload(1, 6, 3, 200, 128, True, seed=77)
    q, k, _ = make_qkv(w)
    _dump_check(w, q, k, [(0, 1)], kv_map=[2, 0, 1, 1, 0, 2])
    w = small_workload(2, 4, 3, 300, 64, False, seed=78)
    q, k, _ = make_qkv(w)
    _dump_check(w, q, k, [(0, 2), (1, 1)], kv_map=[1, 2, 2, 0])


@pytest.mark.parametrize("D,Hkv", [(64, 4), (128, 1)])
def test_int32_scores_two_items_per_workgroup(D, Hkv):
    """Causal launches with at least 8 work items per compute unit give each
    workgroup two items (the schedule of the 1024-token batched MQA and the
    long prefills): every tile of 16 x 16 heads x 1024 tokens, both head dims."""
    w = small_workload(16, 16, Hkv, 1024, D, True, seed=700 + D)
    assert 16 * 16 * 8 >= 8 * torch.cuda.get_device_properties(0).multi_processor_count
    q, k, _ = make_qkv(w)
    _dump_check(w, q, k, [(0, 7)])


# --------------------------------------------------------------------------
# FP16 path
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S", TAILS)
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_tails_d128_gqa(S, causal):
    w = small_workload(1, 4, 2, S, 128, causal, seed=1000 + S)
    q, k, v = make_qkv(w)
    _fp16_check(w, q, k, v)


@pytest.mark.parametrize("S", [1, 2, 15, 16, 17, 64, 65, 128, 129, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_tails_d64_mha(S, causal):
    w = small_workload(2, 3, 3, S, 64, causal, seed=2000 + S)
    q, k, v = make_qkv(w)
    _fp16_check(w, q, k, v)


def test_fp16_mqa_and_explicit_map():
    w = small_workload(1, 8, 1, 333, 128, True, seed=31)
    q, k, v = make_qkv(w)
    _fp16_check(w, q, k, v)
    w2 = small_workload(1, 6, 3, 257, 64, False, seed=32)
    q, k, v = make_qkv(w2)
    _fp16_check(w2, q, k, v, kv_map=[2, 0, 1, 1, 0, 2])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_fp16_workloads_sampled(name):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    rows = None if w.seq <= 256 else sample_rows(w.seq, 24, seed=w.seed)
    _fp16_check(w, q, k, v, rows=rows)


# --------------------------------------------------------------------------
# INT8 path
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S", TAILS)
@pytest.mark.parametrize("causal", [False, True])
def test_int8_tails_d128_gqa(S, causal):
    w = small_workload(1, 4, 2, S, 128, causal, seed=3000 + S)
    q, k, v = make_qkv(w)
    _int8_check(w, q, k, v)


@pytest.mark.parametrize("S", [1, 2, 15, 16, 17, 64, 65, 128, 129, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_int8_tails_d64_mha(S, causal):
    w = small_workload(2, 3, 3, S, 64, causal, seed=4000 + S)
    q, k, v = make_qkv(w)
    _int8_check(w, q, k, v)


def test_int8_mqa_and_explicit_map():
    w = small_workload(1, 8, 1, 333, 128, True, seed=41)
    q, k, v = make_qkv(w)
    _int8_check(w, q, k, v)
    w2 = small_workload(1, 6, 3, 257, 64, False, seed=42)
    q, k, v = make_qkv(w2)
    _int8_check(w2, q, k, v, kv_map=[2, 0, 1, 1, 0, 2])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_int8_workloads_sampled(name):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    rows = None if w.seq <= 256 else sample_rows(w.seq, 24, seed=w.seed)
    _int8_check(w, q, k, v, rows=rows)


def test_fp16_and_int8_at_a_million_tokens_sampled():
    """2^20 tokens, causal, two q-heads on one kv-head, head_dim 64: per-lane
    offsets, tile counts and the two-items-per-workgroup schedule at a long
    sequence; sampled rows against the oracle (FP16 and INT8 paths)."""
    w = small_workload(1, 2, 1, 1 << 20, 64, True, seed=81)
    q, k, v = make_qkv(w)
    rows = sample_rows(w.seq, 8, seed=81)
    _fp16_check(w, q, k, v, rows=rows)
    _int8_check(w, q, k, v, rows=rows)


def test_fp16_and_int8_at_the_maximum_sequence_sampled():
    """ATTN_MAX_SEQ = 2^22 tokens, causal, head_dim 128 (1 GiB per K and V
    head, the largest per-lane copy offsets): sampled rows against the oracle
    (FP16 and INT8 paths)."""
    w = small_workload(1, 1, 1, 1 << 22, 128, True, seed=83)
    q, k, v = make_qkv(w)
    rows = sample_rows(w.seq, 6, seed=83)
    _fp16_check(w, q, k, v, rows=rows)
    _int8_check(w, q, k, v, rows=rows)


# --------------------------------------------------------------------------
# lse, invariants, determinism, wrappers
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_lse_both_paths(causal):
    w = small_workload(1, 4, 2, 300, 128, causal, seed=51)
    q, k, v = make_qkv(w)
    case(f"lse causal={causal}")
    _, lse16 = A.fwd_fp16(dev(q), dev(k), dev(v), causal=causal, return_lse=True)
    qz = A.quantize_qk(dev(q), dev(k))
    _, lse8 = A.fwd_int8(qz, dev(v), causal=causal, return_lse=True)
    torch.cuda.synchronize()
    _, ref = O.attention(q, k, v, causal=causal, with_lse=True)
    assert np.abs(host(lse16) - ref).max() < 1e-3
    qz_h = {key: host(qz[key]) for key in ("q_i8", "q_scale", "k_i8", "k_scale")}
    _, ref8 = O.quant_attention(qz_h, v, causal=causal, with_lse=True)
    assert np.abs(host(lse8) - ref8).max() < 1e-3


@pytest.mark.parametrize("path", ["fp16", "int8"])
def test_constant_v_and_causal_row0(path):
    w = small_workload(1, 4, 2, 777, 128, True, seed=61)
    q, k, v = make_qkv(w)
    c = np.float16(0.3330078125)
    vc = np.full_like(v, c)
    case(f"invariants {path}")
    if path == "fp16":
        out_c = A.fwd_fp16(dev(q), dev(k), dev(vc), causal=True)
        out = A.fwd_fp16(dev(q), dev(k), dev(v), causal=True)
    else:
        qz = A.quantize_qk(dev(q), dev(k))
        out_c = A.fwd_int8(qz, dev(vc), causal=True)
        out = A.fwd_int8(qz, dev(v), causal=True)
    torch.cuda.synchronize()
    assert np.abs(host(out_c).astype(np.float64) - float(c)).max() <= 2.0 ** -11
    o = host(out)
    kv_map = np.arange(4) // 2
    for h in range(4):
        assert np.array_equal(o[0, h, 0], v[0, kv_map[h], 0])


@pytest.mark.parametrize("path", ["fp16", "int8"])
def test_runs_are_bitwise_deterministic(path):
    w = WORKLOADS["batched_mqa"].scaled(batch=4)
    q, k, v = make_qkv(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    case(f"determinism {path}")
    outs = []
    for _ in range(3):
        if path == "fp16":
            outs.append(A.fwd_fp16(qd, kd, vd, causal=True).clone())
        else:
            outs.append(A.fwd_int8(A.quantize_qk(qd, kd), vd, causal=True).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_gqa_equals_mha_on_repeated_kv_gpu():
    w = small_workload(1, 8, 2, 300, 128, True, seed=71)
    q, k, v = make_qkv(w)
    rk, rv = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    case("gqa == mha(repeated) fp16")
    a = A.fwd_fp16(dev(q), dev(k), dev(v), causal=True)
    b = A.fwd_fp16(dev(q), dev(rk), dev(rv), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("D", [64, 128])
def test_causal_future_keys_have_no_effect(D):
    """Causal mask (MHA-GQA article, §2.3): perturbing the keys and values of
    positions after row i leaves rows 0..i bit-identical (FP16 path, whose
    inputs are used as given); the INT8 path is checked with the quantised
    tensors held fixed, so that only the masked products change."""
    S, cut = 300, 173
    w = small_workload(1, 4, 2, S, D, True, seed=91 + D)
    q, k, v = make_qkv(w)
    k2, v2 = k.copy(), v.copy()
    rng = np.random.default_rng(5)
    k2[:, :, cut:] = rng.standard_normal(k2[:, :, cut:].shape).astype(np.float16) * 8
    v2[:, :, cut:] = -v2[:, :, cut:] + 1
    case(f"causal future keys D={D}")
    a = A.fwd_fp16(dev(q), dev(k), dev(v), causal=True)
    b = A.fwd_fp16(dev(q), dev(k2), dev(v2), causal=True)
    qz = A.quantize_qk(dev(q), dev(k))
    qz2 = dict(qz)
    k8 = qz["k_i8"].clone()
    k8[:, :, cut:] = torch.randint(-127, 128, k8[:, :, cut:].shape, dtype=torch.int8, device=k8.device)
    qz2["k_i8"] = k8
    c = A.fwd_int8(qz, dev(v), causal=True)
    d = A.fwd_int8(qz2, dev(v2), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[:, :, :cut], b[:, :, :cut]) and not torch.equal(a, b)
    assert torch.equal(c[:, :, :cut], d[:, :, :cut]) and not torch.equal(c, d)


def test_kv_head_change_reaches_only_its_group():
    """GQA (MHA-GQA article, §5.1): changing K/V of kv-head 1 changes exactly
    the q-heads mapped to it, for the default and an explicit map."""
    w = small_workload(1, 8, 4, 200, 128, False, seed=97)
    q, k, v = make_qkv(w)
    k2, v2 = k.copy(), v.copy()
    k2[:, 1] = k2[:, 1][:, ::-1]
    v2[:, 1] = v2[:, 1] * 2
    for kv_map in (None, [3, 1, 0, 1, 2, 2, 1, 0]):
        case(f"kv-head group isolation map={kv_map}")
        a = host(A.fwd_fp16(dev(q), dev(k), dev(v), kv_head_map=kv_map))
        b = host(A.fwd_fp16(dev(q), dev(k2), dev(v2), kv_head_map=kv_map))
        heads = [h for h in range(8) if (h // 2 if kv_map is None else kv_map[h]) == 1]
        for h in range(8):
            same = np.array_equal(a[:, h], b[:, h])
            assert same == (h not in heads), (kv_map, h)


def test_custom_scale_and_sageattn_wrapper():
    w = small_workload(1, 4, 2, 200, 64, False, seed=81)
    q, k, v = make_qkv(w)
    case("custom scale fp16 / sageattn")
    out = A.fwd_fp16(dev(q), dev(k), dev(v), sm_scale=0.05)
    ref = O.attention(q, k, v, sm_scale=0.05)
    torch.cuda.synchronize()
    assert np.abs(host(out) - ref).max() <= FP16_MAX_ABS
    s = A.sageattn(dev(q), dev(k), dev(v), is_causal=True, scale=0.1)
    qz = A.quantize_qk(dev(q), dev(k))
    t = A.fwd_int8(qz, dev(v), causal=True, sm_scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(s, t)
    cos, rel = cos_rel_l1(host(s), O.attention(q, k, v, causal=True, sm_scale=0.1))
    assert cos >= INT8_COS_MIN and rel <= INT8_REL_L1_MAX


# --------------------------------------------------------------------------
# fused Q quantisation: bitwise the same as quantize_qk + fwd_int8
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S,D,Hq,Hkv,causal", [
    (1, 64, 2, 2, False), (17, 128, 4, 2, True), (127, 64, 3, 3, True), (128, 128, 4, 1, False),
    (129, 128, 8, 2, True), (300, 64, 2, 1, False), (1000, 128, 4, 2, True)])
def test_fused_q_matches_two_call_path_bitwise(S, D, Hq, Hkv, causal):
    w = small_workload(1, Hq, Hkv, S, D, causal, seed=5000 + S + D)
    q, k, v = make_qkv(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    case(f"fused-q S={S} D={D} Hq={Hq} Hkv={Hkv} causal={causal}")
    qz = A.quantize_qk(qd, kd)
    o_ref, lse_ref = A.fwd_int8(qz, vd, causal=causal, return_lse=True)
    kz = A.quantize_k(kd)
    qs = torch.full_like(qz["q_scale"], -1.0)
    o, lse = A.fwd_int8_fused_q(qd, kz, vd, causal=causal, return_lse=True, q_scale_out=qs)
    torch.cuda.synchronize()
    for key in ("k_i8", "k_scale", "k_mean"):
        assert torch.equal(kz[key], qz[key]), key
    assert torch.equal(qs, qz["q_scale"])
    assert torch.equal(o, o_ref)
    assert torch.equal(lse, lse_ref)


@pytest.mark.parametrize("name", ["llm_prefill_gqa", "batched_mqa", "video_mha", "long_gqa"])
def test_fused_q_workloads_bitwise_and_accuracy(name):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    case(f"fused-q workload {name}")
    qz = A.quantize_qk(qd, kd)
    o_ref = A.fwd_int8(qz, vd, causal=w.causal)
    o = A.sageattn(qd, kd, vd, is_causal=w.causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    rows = sample_rows(w.seq, 16, seed=w.seed + 7)
    cos, rel = cos_rel_l1(host(o)[:, :, rows], O.attention(q, k, v, causal=w.causal, rows=rows))
    assert cos >= INT8_COS_MIN and rel <= INT8_REL_L1_MAX, (cos, rel)


def _random_configs(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8]))
        mapped = bool(rng.integers(0, 2)) and group > 1
        out.append(dict(B=int(rng.integers(1, 4)), Hq=hkv * group, Hkv=hkv, S=int(rng.integers(1, 1501)),
                        D=int(rng.choice([64, 128])), causal=bool(rng.integers(0, 2)), mapped=mapped,
                        seed=3000 + i))
    return out


@pytest.mark.parametrize("cfg", _random_configs(), ids=lambda c: "B{B}-H{Hq}x{Hkv}-S{S}-D{D}-{c}{m}".format(
    c="causal" if c["causal"] else "full", m="-map" if c["mapped"] else "", **c))
def test_random_shapes_fp16_int8_fused(cfg):
    """Seeded random shapes (batch, GQA groups, explicit maps, any length up to
    1500, both head dims, both masks): FP16 and INT8 paths against the oracle on
    up to 96 rows, and the fused-Q path bit for bit against the two-call path."""
    w = small_workload(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"], cfg["causal"], cfg["seed"])
    q, k, v = make_qkv(w)
    kv_map = None
    if cfg["mapped"]:
        kv_map = [int(x) for x in np.random.default_rng(cfg["seed"]).integers(0, cfg["Hkv"], cfg["Hq"])]
    S = cfg["S"]
    rng = np.random.default_rng(cfg["seed"] + 1)
    rows = np.unique(np.r_[0, S - 1, rng.integers(0, S, min(S, 94))]) if S > 96 else None
    _fp16_check(w, q, k, v, rows=rows, kv_map=kv_map)
    _int8_check(w, q, k, v, rows=rows, kv_map=kv_map)
    case(f"fused vs two-call {w.name} map={kv_map}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    qz = A.quantize_qk(qd, kd)
    a = A.fwd_int8(qz, vd, causal=w.causal, kv_head_map=kv_map)
    b = A.fwd_int8_fused_q(qd, A.quantize_k(kd), vd, causal=w.causal, kv_head_map=kv_map)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
