"""Pins of the oracle's tile-masked attention (the APB page: a FlashAttention
kernel with a changed attention-mask shape; on one device the keys are the
anchor block, the passing block and the local context, in that order).

Mask entry (query tile of 128 rows, key tile of 64 keys): 0 invisible,
1 visible, 2 visible iff key j <= query i.  Pinned by: the causal and the
full mask written as tile masks (against the square oracle), a local-window
mask (against independent per-chunk causal attention), the APB layout
(against causal attention, with the passing rows empty) and random masks
(against torch's float64 scaled_dot_product_attention with a boolean mask).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O

TQ, TK = O.TILE_Q, O.TILE_K


def _f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def _inputs(S, D=32, Hq=4, Hkv=2, seed=0):
    rng = np.random.default_rng(seed)
    q = _f16(rng, (1, Hq, S, D))
    k = (rng.standard_normal((1, Hkv, S, D)) + rng.standard_normal(D) * 2).astype(np.float16)
    v = _f16(rng, (1, Hkv, S, D))
    return q, k, v


def causal_tile_mask(S):
    nqt, nkt = -(-S // TQ), -(-S // TK)
    m = np.zeros((nqt, nkt), np.uint8)
    for qt in range(nqt):
        for kt in range(nkt):
            if kt * TK + TK - 1 <= qt * TQ:
                m[qt, kt] = 1           # every key of the tile precedes every query of the q-tile
            elif kt * TK <= min(S - 1, qt * TQ + TQ - 1):
                m[qt, kt] = 2           # the tile crosses the diagonal
    return m


def apb_tile_mask(anchor, passing, local):
    """Keys [anchor | passing | local]; anchor rows causal over the anchor,
    local rows see anchor and passing fully and the local block causally,
    rows at passing positions see nothing."""
    S = anchor + passing + local
    c = causal_tile_mask(S)
    m = c.copy()
    q0p, q1p = anchor // TQ, (anchor + passing) // TQ
    m[q0p:q1p, :] = 0
    return m


@pytest.mark.parametrize("S", [1, 64, 129, 300])
def test_causal_as_tile_mask_equals_causal(S):
    q, k, v = _inputs(S, seed=S)
    a, la = O.attention_masked(q, k, v, causal_tile_mask(S), with_lse=True)
    b, lb = O.attention(q, k, v, causal=True, with_lse=True)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)


def test_full_mask_equals_non_causal():
    q, k, v = _inputs(200, seed=3)
    m = np.ones((2, 4), np.uint8)
    np.testing.assert_allclose(O.attention_masked(q, k, v, m), O.attention(q, k, v), rtol=0, atol=1e-13)


def test_local_window_equals_per_chunk_causal():
    """Each query tile sees only its own diagonal key tiles (causally): the
    result is causal attention inside each 128-row chunk, computed here as
    separate problems."""
    S = 384
    q, k, v = _inputs(S, seed=4)
    m = np.zeros((3, 6), np.uint8)
    for qt in range(3):
        m[qt, 2 * qt] = m[qt, 2 * qt + 1] = 2
    got = O.attention_masked(q, k, v, m)
    for c in range(3):
        sl = slice(c * TQ, (c + 1) * TQ)
        ref = O.attention(np.ascontiguousarray(q[:, :, sl]), np.ascontiguousarray(k[:, :, sl]),
                          np.ascontiguousarray(v[:, :, sl]), causal=True)
        np.testing.assert_allclose(got[:, :, sl], ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("anchor,passing,local", [(128, 128, 256), (256, 384, 128), (128, 256, 200)])
def test_apb_mask_is_causal_without_the_passing_rows(anchor, passing, local):
    S = anchor + passing + local
    q, k, v = _inputs(S, seed=anchor + passing)
    got, gl = O.attention_masked(q, k, v, apb_tile_mask(anchor, passing, local), with_lse=True)
    ref, rl = O.attention(q, k, v, causal=True, with_lse=True)
    keep = np.r_[0:anchor, anchor + passing:S]
    np.testing.assert_allclose(got[:, :, keep], ref[:, :, keep], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gl[:, :, keep], rl[:, :, keep], rtol=0, atol=1e-12)
    assert not got[:, :, anchor:anchor + passing].any()
    assert np.all(np.isneginf(gl[:, :, anchor:anchor + passing]))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_masks_against_torch_sdpa(seed):
    S, D = 257, 16
    q, k, v = _inputs(S, D=D, Hq=2, Hkv=1, seed=10 + seed)
    rng = np.random.default_rng(seed)
    m = rng.integers(0, 3, (-(-S // TQ), -(-S // TK))).astype(np.uint8)
    got = O.attention_masked(q, k, v, m)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    t = m[i // TQ, j // TK]
    vis = (t == 1) | ((t == 2) & (j <= i))
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(np.repeat(k, 2, axis=1).astype(np.float64))
    vt = torch.from_numpy(np.repeat(v, 2, axis=1).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(vis)).numpy()
    rows = vis.any(axis=1)
    np.testing.assert_allclose(got[:, :, rows], ref[:, :, rows], rtol=0, atol=1e-12)
    assert not got[:, :, ~rows].any()


def test_quant_masked_with_causal_mask_equals_quant_causal():
    S = 300
    q, k, v = _inputs(S, D=64, seed=20)
    qz = O.quantize_qk(q, k)
    a = O.quant_attention_masked(qz, v, causal_tile_mask(S))
    b = O.quant_attention(qz, v, causal=True)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_quant_masked_apb_rows():
    q, k, v = _inputs(512, D=64, seed=21)
    qz = O.quantize_qk(q, k)
    got = O.quant_attention_masked(qz, v, apb_tile_mask(128, 128, 256))
    ref = O.quant_attention(qz, v, causal=True)
    keep = np.r_[0:128, 256:512]
    np.testing.assert_allclose(got[:, :, keep], ref[:, :, keep], rtol=0, atol=1e-13)
    assert not got[:, :, 128:256].any()
