"""GPU parity of the tile-masked forward (the APB page's FlashAttention kernel
with a changed mask shape) against the CPU oracle.

* attn_fwd_fp16_masked: max-abs <= 2e-3 against the oracle's exact masked
  attention; rows with no visible key give O = 0 and lse = -inf exactly.
* attn_fwd_int8_masked: max-abs <= 2e-3 against the oracle's masked
  quantised model; cosine / relative-L1 bars against exact masked attention.
* The causal mask written as a tile mask, and the APB mask outside the
  passing rows, reproduce the causal kernels bit for bit (same tiles in the
  same order; the extra fully masked tiles add exact zeros).
* Random masks (with empty rows and sequence tails), GQA maps, both head
  dims, and a full-size APB prefill.
"""
import numpy as np
import pytest
import torch

import bit_quantized_exact_amd as A
from bit_quantized_exact_amd.inputs import WORKLOADS, make_qkv
from oracle import oracle as O

from _util import (FP16_MAX_ABS, INT8_COS_MIN, INT8_REL_L1_MAX, INT8_VS_MODEL_MAX_ABS, case, cos_rel_l1, dev,
                   host, small_workload)

pytestmark = pytest.mark.gpu


def _causal_mask(S):
    nq, nk = A.block_mask_tiles(S)
    i0 = np.arange(nq)[:, None] * 128
    j0 = np.arange(nk)[None, :] * 64
    return np.where(j0 + 63 <= i0, 1, np.where(j0 <= np.minimum(S - 1, i0 + 127), 2, 0)).astype(np.uint8)


def _check(w, q, k, v, mask, kv_map=None, rows=None):
    S = w.seq
    csr = A.block_mask_csr(S, mask)
    case(f"fwd_fp16_masked {w.name} S={S} D={w.head_dim} nnz={csr['nnz']} map={kv_map}")
    o16, l16 = A.fwd_fp16_masked(dev(q), dev(k), dev(v), csr, kv_head_map=kv_map, return_lse=True)
    case(f"fwd_int8_masked {w.name}")
    qz = A.quantize_qk(dev(q), dev(k))
    o8, l8 = A.fwd_int8_masked(qz, dev(v), csr, kv_head_map=kv_map, return_lse=True)
    torch.cuda.synchronize()
    g16, g8 = host(o16).astype(np.float64), host(o8).astype(np.float64)
    gl16, gl8 = host(l16).astype(np.float64), host(l8).astype(np.float64)
    exact, el = O.attention_masked(q, k, v, mask, kv_map=kv_map, with_lse=True)
    qz_h = {key: host(qz[key]) for key in ("q_i8", "q_scale", "k_i8", "k_scale")}
    model, ml = O.quant_attention_masked(qz_h, v, mask, kv_map=kv_map, with_lse=True)
    sel = (slice(None), slice(None), rows if rows is not None else slice(None))
    empty = np.isneginf(el)
    # rows without a visible key: exactly zero and -inf
    assert not g16[empty].any() and not g8[empty].any()
    assert np.all(np.isneginf(gl16[empty])) and np.all(np.isneginf(gl8[empty]))
    full = ~empty
    assert np.abs(g16 - exact)[sel].max() <= FP16_MAX_ABS
    assert np.abs(g8 - model)[sel].max() <= INT8_VS_MODEL_MAX_ABS
    if full.any():
        assert np.abs(gl16[full] - el[full]).max() <= 1e-3
        assert np.abs(gl8[full] - ml[full]).max() <= 1e-4
        cos, rel = cos_rel_l1(g8[full], exact[full])
        assert cos >= INT8_COS_MIN and rel <= INT8_REL_L1_MAX, (cos, rel)
    return o16, o8, qz


@pytest.mark.parametrize("S,D", [(1, 64), (200, 128), (513, 64), (1000, 128)])
def test_causal_tile_mask_is_bitwise_the_causal_kernel(S, D):
    w = small_workload(1, 4, 2, S, D, True, 500 + S)
    q, k, v = make_qkv(w)
    o16, o8, qz = _check(w, q, k, v, _causal_mask(S))
    c16 = A.fwd_fp16(dev(q), dev(k), dev(v), causal=True)
    c8 = A.fwd_int8(qz, dev(v), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o16, c16) and torch.equal(o8, c8)


@pytest.mark.parametrize("anchor,passing,local,D", [(128, 256, 384, 128), (256, 128, 333, 64)])
def test_apb_mask(anchor, passing, local, D):
    S = anchor + passing + local
    w = small_workload(1, 8, 2, S, D, False, 600 + S)
    q, k, v = make_qkv(w)
    m = A.apb_block_mask(S, anchor, passing)
    o16, o8, qz = _check(w, q, k, v, m)
    c16 = A.fwd_fp16(dev(q), dev(k), dev(v), causal=True)
    c8 = A.fwd_int8(qz, dev(v), causal=True)
    torch.cuda.synchronize()
    keep = torch.from_numpy(np.r_[0:anchor, anchor + passing:S]).cuda()
    assert torch.equal(o16[:, :, keep], c16[:, :, keep]) and torch.equal(o8[:, :, keep], c8[:, :, keep])


@pytest.mark.parametrize("S,D,seed,kv_map", [(129, 64, 0, None), (300, 128, 1, None), (700, 64, 2, [1, 0, 1, 1]),
                                             (1025, 128, 3, None)])
def test_random_masks(S, D, seed, kv_map):
    w = small_workload(1, 4, 2, S, D, False, 700 + seed)
    q, k, v = make_qkv(w)
    nq, nk = A.block_mask_tiles(S)
    m = np.random.default_rng(seed).integers(0, 3, (nq, nk)).astype(np.uint8)
    m[min(1, nq - 1), :] = 0           # one query tile with no visible key at all
    _check(w, q, k, v, m, kv_map=kv_map)


def test_empty_mask_gives_zero_rows():
    w = small_workload(1, 2, 1, 300, 64, False, 800)
    q, k, v = make_qkv(w)
    nq, nk = A.block_mask_tiles(300)
    _check(w, q, k, v, np.zeros((nq, nk), np.uint8))


def test_apb_prefill_full_size_sampled():
    """The LLM-prefill shape (32/8 heads, D=128, 8192 tokens) as APB: 1024
    anchor tokens, 2048 passing, 5120 local; sampled rows against the oracle."""
    base = WORKLOADS["llm_prefill_gqa"]
    w = base.scaled(causal=False)
    q, k, v = make_qkv(w)
    m = A.apb_block_mask(w.seq, 1024, 2048)
    rows = np.r_[0, 1, 127, 128, 1023, 1024, 3071, 3072, 3073, 5000, 8191]
    csr = A.block_mask_csr(w.seq, m)
    case("fwd_fp16_masked / fwd_int8_masked full-size APB")
    o16 = A.fwd_fp16_masked(dev(q), dev(k), dev(v), csr)
    qz = A.quantize_qk(dev(q), dev(k))
    o8 = A.fwd_int8_masked(qz, dev(v), csr)
    torch.cuda.synchronize()
    # the sampled rows' reference: exact attention over each row's visible keys
    exact = O.attention(q, k, v, causal=True, rows=rows)
    passing = (rows >= 1024) & (rows < 3072)
    exact[:, :, passing] = 0.0
    g16 = host(o16).astype(np.float64)[:, :, rows]
    g8 = host(o8).astype(np.float64)[:, :, rows]
    assert np.abs(g16 - exact).max() <= FP16_MAX_ABS
    assert not g8[:, :, passing].any()
    cos, rel = cos_rel_l1(g8[:, :, ~passing], exact[:, :, ~passing])
    assert cos >= INT8_COS_MIN and rel <= INT8_REL_L1_MAX, (cos, rel)


@pytest.mark.parametrize("S", [32768, 32769])
def test_apb_mask_long_lists(S):
    """Key-tile lists of up to 512 tiles are copied into LDS and staged
    directly (S = 32768); longer ones (S = 32769: 513 key tiles) are read from
    global memory on the register-staged path.  Both must reproduce the causal
    kernel bit for bit outside the passing rows and give zero rows inside."""
    anchor, passing = 1024, 2048
    w = small_workload(1, 2, 1, S, 64, False, 900 + S % 7)
    q, k, v = make_qkv(w)
    m = A.apb_block_mask(S, anchor, passing)
    csr = A.block_mask_csr(S, m)
    case(f"fwd_*_masked long list S={S} nnz={csr['nnz']}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    o16 = A.fwd_fp16_masked(qd, kd, vd, csr)
    qz = A.quantize_qk(qd, kd)
    o8 = A.fwd_int8_masked(qz, vd, csr)
    c16 = A.fwd_fp16(qd, kd, vd, causal=True)
    c8 = A.fwd_int8(qz, vd, causal=True)
    torch.cuda.synchronize()
    keep = torch.from_numpy(np.r_[0:anchor, anchor + passing:S]).cuda()
    assert torch.equal(o16[:, :, keep], c16[:, :, keep]) and torch.equal(o8[:, :, keep], c8[:, :, keep])
    assert not o16[:, :, anchor:anchor + passing].any() and not o8[:, :, anchor:anchor + passing].any()
    # a few rows against the oracle (exact causal attention over the visible keys)
    rows = np.r_[0, anchor - 1, anchor + passing, S // 2, S - 1]
    exact = O.attention(q, k, v, causal=True, rows=rows)
    assert np.abs(host(o16).astype(np.float64)[:, :, rows] - exact).max() <= FP16_MAX_ABS


@pytest.mark.parametrize("S,D,Hq,Hkv", [(1024, 128, 16, 4), (1000, 64, 20, 5)])
def test_two_items_per_workgroup_is_bitwise_the_one_item_kernel(S, D, Hq, Hkv):
    """Causal launches with at least 8 (batch, head, query tile) items per
    compute unit run two items per workgroup (snake schedule); the tile-mask
    kernel, which keeps one item per workgroup, computes the same tiles in
    the same order, so the outputs and lse must agree bit for bit.  The batch
    is sized from the device's compute-unit count so that the two-item path is
    the one taken; the item count is not a multiple of 8 either."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nqt = (S + 127) // 128
    B = (8 * cus) // (Hq * nqt) + 1
    items = B * Hq * nqt
    assert items >= 8 * cus
    w = small_workload(B, Hq, Hkv, S, D, True, 900 + S)
    q, k, v = make_qkv(w)
    csr = A.block_mask_csr(S, _causal_mask(S))
    case(f"two items per workgroup: B={B} Hq={Hq} S={S} D={D} items={items} cus={cus}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    c16, cl16 = A.fwd_fp16(qd, kd, vd, causal=True, return_lse=True)
    m16, ml16 = A.fwd_fp16_masked(qd, kd, vd, csr, return_lse=True)
    qz = A.quantize_qk(qd, kd)
    c8, cl8 = A.fwd_int8(qz, vd, causal=True, return_lse=True)
    m8, ml8 = A.fwd_int8_masked(qz, vd, csr, return_lse=True)
    f8 = A.fwd_int8_fused_q(qd, A.quantize_k(kd), vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(c16, m16) and torch.equal(cl16, ml16)
    assert torch.equal(c8, m8) and torch.equal(cl8, ml8)
    assert torch.equal(f8, c8)
    # and a sampled check against the oracle (rows of the first and last head)
    rows = np.r_[0:3, S // 2, S - 1]
    exact = O.attention(q[:1, :1], k[:1, :1], v[:1, :1], causal=True, rows=rows)
    assert np.abs(host(c16)[:1, :1, rows].astype(np.float64) - exact).max() <= FP16_MAX_ABS


@pytest.mark.parametrize("S,D,Hq,Hkv,kv_map", [(700, 128, 8, 2, None), (1024, 64, 12, 3, [2, 0, 1] * 4)])
def test_results_do_not_depend_on_the_launch_size(S, D, Hq, Hkv, kv_map):
    """A batch large enough for two items per workgroup gives, for its first
    and last sequence, bit for bit what a launch of that sequence alone (one
    item per workgroup) gives: FP16, two-call INT8 and fused INT8 forwards,
    outputs and lse, under an explicit kv-head map too."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nqt = (S + 127) // 128
    B = (8 * cus) // (Hq * nqt) + 2
    w = small_workload(B, Hq, Hkv, S, D, True, 950 + S)
    q, k, v = make_qkv(w)
    case(f"launch-size invariance: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} map={kv_map} cus={cus}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    kz = A.quantize_k(kd)
    qz = A.quantize_qk(qd, kd)

    def run(sl):
        qs, ks, vs = qd[sl].contiguous(), kd[sl].contiguous(), vd[sl].contiguous()
        kzs = {key: (t[sl].contiguous() if isinstance(t, torch.Tensor) and t.dim() > 1 else t) for key, t in kz.items()}
        qzs = {key: (t[sl].contiguous() if isinstance(t, torch.Tensor) and t.dim() > 1 else t) for key, t in qz.items()}
        o16, l16 = A.fwd_fp16(qs, ks, vs, causal=True, kv_head_map=kv_map, return_lse=True)
        o8, l8 = A.fwd_int8(qzs, vs, causal=True, kv_head_map=kv_map, return_lse=True)
        f8, fl8 = A.fwd_int8_fused_q(qs, kzs, vs, causal=True, kv_head_map=kv_map, return_lse=True)
        return [o16, l16, o8, l8, f8, fl8]

    full = run(slice(0, B))
    for b in (0, B - 1):
        one = run(slice(b, b + 1))
        torch.cuda.synchronize()
        for x, y in zip(full, one):
            assert torch.equal(x[b:b + 1], y)
