"""Host helpers of the tile-mask forward (no GPU): the APB layout builder and
the dense-mask -> tile-list conversion the kernels read.

The list is checked semantically: decoding it back into the per-(query, key)
visibility relation must give exactly the relation of the dense mask (tile
types 0 none, 1 all, 2 key j <= query i).
"""
import ctypes

import numpy as np
import pytest

import bit_quantized_exact_amd as A

TQ, TK = 128, 64


def _visibility_dense(seq, mask):
    i = np.arange(seq)[:, None]
    j = np.arange(seq)[None, :]
    t = mask[i // TQ, j // TK]
    return (t == 1) | ((t == 2) & (j <= i))


def _visibility_list(seq, row_ptr, cols):
    vis = np.zeros((seq, seq), bool)
    for qt in range(len(row_ptr) - 1):
        i0, i1 = qt * TQ, min(seq, qt * TQ + TQ)
        for e in cols[row_ptr[qt]:row_ptr[qt + 1]]:
            kt, ty = int(e) >> 2, int(e) & 3
            j0, j1 = kt * TK, min(seq, kt * TK + TK)
            for i in range(i0, i1):
                if ty == 1:
                    vis[i, j0:j1] = True
                elif ty == 2:
                    vis[i, j0:min(j1, i + 1)] = True
    return vis


def _csr_host(seq, mask):
    nq, nk = A.block_mask_tiles(seq)
    rp = np.zeros(nq + 1, np.int32)
    cols = np.zeros(nq * nk, np.int32)
    nnz = ctypes.c_int32()
    st = A.lib().attn_block_mask_csr(seq, np.ascontiguousarray(mask, np.uint8).ctypes.data_as(ctypes.c_void_p),
                                     rp.ctypes.data_as(ctypes.c_void_p), cols.ctypes.data_as(ctypes.c_void_p),
                                     ctypes.byref(nnz))
    return st, rp, cols[:nnz.value]


def test_tile_counts():
    assert A.block_mask_tiles(1) == (1, 1)
    assert A.block_mask_tiles(128) == (1, 2)
    assert A.block_mask_tiles(129) == (2, 3)
    assert A.lib().attn_block_mask_tiles(0, None, None) == -1


@pytest.mark.parametrize("anchor,passing,seq", [(128, 128, 512), (256, 384, 896), (0, 128, 300), (128, 0, 200),
                                                (128, 256, 384)])
def test_apb_builder_matches_its_definition(anchor, passing, seq):
    m = A.apb_block_mask(seq, anchor, passing)
    vis = _visibility_dense(seq, m)
    i = np.arange(seq)[:, None]
    j = np.arange(seq)[None, :]
    passing_row = (i >= anchor) & (i < anchor + passing)
    want = (j <= i) & ~passing_row          # causal over [anchor|passing|local], passing rows empty
    assert np.array_equal(vis, want)


@pytest.mark.parametrize("args", [(300, 100, 128), (300, 128, 100), (300, 256, 128), (0, 0, 0), (300, -128, 0)])
def test_apb_builder_rejects_misaligned_blocks(args):
    seq, anchor, passing = args
    buf = np.zeros(64, np.uint8)
    assert A.lib().attn_block_mask_apb(seq, anchor, passing, buf.ctypes.data_as(ctypes.c_void_p)) == -1


@pytest.mark.parametrize("seq,seed", [(1, 0), (64, 1), (129, 2), (300, 3), (1000, 4)])
def test_list_encodes_the_same_relation(seq, seed):
    nq, nk = A.block_mask_tiles(seq)
    m = np.random.default_rng(seed).integers(0, 3, (nq, nk)).astype(np.uint8)
    st, rp, cols = _csr_host(seq, m)
    assert st == 0
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == len(cols)
    for qt in range(nq):                         # key order, in-range tiles, types 1/2 only
        kts = cols[rp[qt]:rp[qt + 1]] >> 2
        assert np.all(np.diff(kts) > 0) and np.all((kts >= 0) & (kts < nk))
    assert np.all(np.isin(cols & 3, [1, 2]))
    assert np.array_equal(_visibility_list(seq, rp, cols), _visibility_dense(seq, m))


def test_list_drops_and_promotes_diagonal_tiles():
    seq = 256
    m = np.full((2, 4), 2, np.uint8)
    st, rp, cols = _csr_host(seq, m)
    # query tile 0 (rows 0..127): key tiles 0, 1 cross the diagonal, 2, 3 lie above it (dropped)
    assert list(cols[rp[0]:rp[1]]) == [(0 << 2) | 2, (1 << 2) | 2]
    # query tile 1 (rows 128..255): key tiles 0, 1 lie below it (become 1), 2, 3 cross it
    assert list(cols[rp[1]:rp[2]]) == [(0 << 2) | 1, (1 << 2) | 1, (2 << 2) | 2, (3 << 2) | 2]


def test_list_rejects_bad_values():
    m = np.full((1, 2), 3, np.uint8)
    st, _, _ = _csr_host(100, m)
    assert st == -1


def test_masked_forward_validation():
    L = A.lib()
    sh = A.AttnShape(1, 4, 2, 256, 128)
    F, M = 0x10000, 0x10008
    P = ctypes.byref(sh)
    assert L.attn_fwd_fp16_masked(P, F, F, F, F, None, None, None, F, 1, 0.0, None) == -1     # no row_ptr
    assert L.attn_fwd_fp16_masked(P, F, F, F, F, None, None, F, None, 1, 0.0, None) == -1     # entries but no list
    assert L.attn_fwd_fp16_masked(P, F, F, F, F, None, None, F, F, -1, 0.0, None) == -1       # negative count
    assert L.attn_fwd_fp16_masked(P, M, F, F, F, None, None, F, F, 1, 0.0, None) == -1
    assert L.attn_fwd_fp16_masked(P, F, F, F, F, None, None, F + 2, F, 1, 0.0, None) == -1
    assert L.attn_fwd_int8_masked(P, F, F, F, F, F, F, None, None, F, F, 1, float("nan"), None) == -1
    assert L.attn_fwd_int8_masked(P, F, None, F, F, F, F, None, None, F, F, 1, 0.0, None) == -1
    bad = A.AttnShape(1, 4, 2, 256, 96)
    assert L.attn_fwd_int8_masked(ctypes.byref(bad), F, F, F, F, F, F, None, None, F, F, 1, 0.0, None) == -2
