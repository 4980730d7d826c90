"""Pins of the oracle's FP8 (E4M3) alternative and of its 8-bit P.V model (O5).

Source: SageAttention article ("又快又准，即插即用！清华8比特量化Attention…"),
section 技术方案: INT8 quantisation of Q and K is more accurate than FP8, and
quantising P and V to 8 bits (INT8, E4M3, E5M2) leaves some layers with poor
accuracy.  The pages print neither the FP8 format details nor the scaling;
the readings (OCP E4M3, per-block absmax scaled to 448, nearest-even, 8-bit
P as E4M3(448 p) / 448 against the online softmax's running maximum, 8-bit V
with one scale per channel) are pinned here against torch's independent
float8_e4m3fn conversion, exact grids, closed forms and error bounds.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O


def _torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_round32(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).double().numpy()


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


# --------------------------------------------------------------------------
# the E4M3 format
# --------------------------------------------------------------------------
def test_decode_every_code_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = O.e4m3_decode(codes), _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert sorted(np.flatnonzero(nan)) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[~nan].max() == 448.0 and ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6


def test_encode_inverts_decode():
    for c in _finite_codes():
        assert O.e4m3_encode(O.e4m3_decode(np.array([c]))[0]) == c


def test_round_every_fp16_value_in_range_against_torch():
    x = np.arange(0x10000, dtype=np.uint16).view(np.float16).astype(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    ours, ref = O.e4m3_round(x), _torch_round32(x)
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_round_random_fp32_against_torch():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), 200000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    assert np.array_equal(O.e4m3_round(x), _torch_round32(x))


def test_round_half_way_cases_go_to_even_codes():
    pos = np.unique(_torch_decode(_finite_codes()))
    pos = pos[pos >= 0]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)     # exact in fp32
    r = O.e4m3_round(mids)
    for m_, v in zip(mids, r):
        c = O.e4m3_encode(v)
        assert c & 1 == 0, (m_, v, c)
        assert v in (pos[pos < m_].max(), pos[pos > m_].min())


def test_round_saturates_and_keeps_the_sign_of_zero():
    assert O.e4m3_round(470.0)[()] == 448.0          # would round to 480, beyond the format
    assert O.e4m3_round(-470.0)[()] == -448.0
    assert O.e4m3_round(460.0)[()] == 448.0          # nearest is 448 itself
    z = O.e4m3_round(np.array([-1e-9, 1e-9]))
    assert z[0] == 0 and np.signbit(z[0]) and not np.signbit(z[1])
    assert O.e4m3_encode(-0.0) == 0x80 and O.e4m3_encode(0.0) == 0


# --------------------------------------------------------------------------
# FP8 block quantisation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S,block", [(200, 64), (128, 128), (1, 64)])
def test_quant_blocks_e4m3_invariants(S, block):
    rng = np.random.default_rng(S + block)
    x = (rng.standard_normal((3, S, 32)) * rng.uniform(0.01, 20, (3, 1, 1))).astype(np.float32)
    codes, sc = O.quant_blocks_e4m3(x, block)
    val = O.e4m3_decode(codes)
    for m in range(3):
        for b in range((S + block - 1) // block):
            xb = x[m, b * block:(b + 1) * block]
            cb = codes[m, b * block:(b + 1) * block]
            a = np.float32(np.abs(xb).max())
            assert sc[m, b] == np.float32(a / np.float32(448.0))
            r = np.float32(np.float32(448.0) / a)
            # the E4M3 step is torch's independent conversion of the fp32 product
            t = np.clip(xb * r, np.float32(-448), np.float32(448)).astype(np.float32)
            assert np.array_equal(O.e4m3_decode(cb), _torch_round32(t))
            # the largest magnitude lands on +-448
            i = np.unravel_index(np.abs(xb).argmax(), xb.shape)
            assert abs(O.e4m3_decode(cb[i][None])[0]) == 448.0
            # half an ulp: 2^-4 relative for normals, 2^-10 absolute below 2^-6 (code units)
            vb = val[m, b * block:(b + 1) * block]
            err = np.abs(vb - t.astype(np.float64))
            assert np.all(err <= np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-12))


def test_quant_blocks_e4m3_zero_block_and_symmetry():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 128, 16)).astype(np.float32)
    x[0, 64:] = 0
    c, sc = O.quant_blocks_e4m3(x, 64)
    assert sc[0, 1] == 0 and not c[0, 64:].any()
    cn, scn = O.quant_blocks_e4m3(-x[:, :64], 64)
    assert scn[0, 0] == sc[0, 0]
    assert np.array_equal(cn[0], c[0, :64] ^ 0x80)


def test_quant_blocks_e4m3_power_of_two_scale_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 100, 16)).astype(np.float32)
    c1, s1 = O.quant_blocks_e4m3(x, 64)
    c2, s2 = O.quant_blocks_e4m3(x * np.float32(8.0), 64)
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * np.float32(8.0))


def test_quant_v_is_per_channel_over_all_tokens():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((1, 2, 100, 16)) * np.linspace(0.1, 5, 16)).astype(np.float16)
    codes, sc = O.quant_v_fp8(v)
    vf = v.astype(np.float64)
    a = np.abs(vf).max(axis=2)                                  # [B, Hkv, D]
    assert np.array_equal(sc, (a.astype(np.float32) / np.float32(448)).astype(np.float32))
    dec = O.e4m3_decode(codes)
    for h in range(2):
        for c in range(16):
            assert np.abs(dec[0, h, :, c]).max() == 448.0
    # per-channel scaling: each channel's error is relative to its own range
    err = np.abs(dec * sc[:, :, None, :] - vf)
    assert np.all(err <= np.maximum(np.abs(vf) * 2.0 ** -4, sc[:, :, None, :] * 2.0 ** -10) * (1 + 1e-6))


# --------------------------------------------------------------------------
# inputs on an exact E4M3 grid (quantisation is then lossless)
# --------------------------------------------------------------------------
def _grid_values(rng, shape, top_index):
    """E4M3 values (torch's decoding of random finite codes) with +448 at top_index."""
    codes = rng.choice(_finite_codes(), size=shape)
    x = _torch_decode(codes)
    x[top_index] = 448.0
    return x


def _lossless_fp8_inputs(rng, S, D, Hq, Hkv, bq, bk):
    q = np.zeros((1, Hq, S, D))
    for h in range(Hq):
        for b0 in range(0, S, bq):
            n = min(bq, S - b0)
            q[0, h, b0:b0 + n] = _grid_values(rng, (n, D), (0, 0)) * 2.0 ** -(8 + (b0 // bq + h) % 3)
    assert S % (2 * bk) == 0 and (S // 2 // bk) % 4 == 0
    k = np.zeros((1, Hkv, S, D))
    half = S // 2
    for h in range(Hkv):
        g = np.zeros((half, D))
        for b0 in range(0, half, bk):
            g[b0:b0 + bk] = _grid_values(rng, (bk, D), (0, 0))
        k[0, h, :half] = g
        k[0, h, half:] = -g                       # channel sums exactly zero
        for b0 in range(0, S, bk):
            k[0, h, b0:b0 + bk] *= 2.0 ** -(7 + (b0 // bk) % 4)
    return q.astype(np.float16), k.astype(np.float16)


def _lossless_v(rng, Hkv, S, D):
    v = np.zeros((1, Hkv, S, D))
    for h in range(Hkv):
        g = _grid_values(rng, (S, D), (0, 0))
        g[0, :] = 448.0 * rng.choice([-1.0, 1.0], D)           # every channel reaches 448
        v[0, h] = g * 2.0 ** -(7 + h)
    return v.astype(np.float16)


@pytest.mark.parametrize("causal", [False, True])
def test_lossless_grid_fp8_dequantisation(causal):
    rng = np.random.default_rng(51)
    S, D, Hq, Hkv = 512, 64, 4, 2
    q, k = _lossless_fp8_inputs(rng, S, D, Hq, Hkv, O.BQ, O.BK)
    assert np.array_equal(q.astype(np.float64).astype(np.float16), q)
    v = (rng.standard_normal((1, Hkv, S, D))).astype(np.float16)
    qz = O.quantize_qk_fp8(q, k)
    assert not qz["k_mean"].any()
    dq = np.repeat(qz["q_scale"], O.BQ, axis=-1)[..., :S, None].astype(np.float64)
    dk = np.repeat(qz["k_scale"], O.BK, axis=-1)[..., :S, None].astype(np.float64)
    assert np.array_equal(_torch_decode(qz["q_f8"]) * dq, q.astype(np.float64))
    assert np.array_equal(_torch_decode(qz["k_f8"]) * dk, k.astype(np.float64))
    o_exact, lse_exact = O.attention(q, k, v, causal=causal, with_lse=True)
    o_q, lse_q = O.quant_attention_fp8(qz, v, causal=causal, with_lse=True)
    np.testing.assert_allclose(lse_q, lse_exact, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_q, o_exact, rtol=0, atol=2e-3)


# --------------------------------------------------------------------------
# O5: 8-bit P and V inside the online softmax
# --------------------------------------------------------------------------
def _int8_lossless(rng, S, D, Hq, Hkv):
    # INT8 lossless grid: integer multiples of a power-of-two step, +-127 per block,
    # zero channel means (the construction of the INT8 pins)
    q = np.zeros((1, Hq, S, D))
    for h in range(Hq):
        for b0 in range(0, S, O.BQ):
            n = min(O.BQ, S - b0)
            blk = rng.integers(-127, 128, (n, D)).astype(np.float64)
            blk[0, 0] = 127
            q[0, h, b0:b0 + n] = blk * 2.0 ** -(4 + (b0 // O.BQ + h) % 3)
    k = np.zeros((1, Hkv, S, D))
    half = S // 2
    for h in range(Hkv):
        ints = rng.integers(-127, 128, (half, D)).astype(np.float64)
        ints[::O.BK, 0] = -127
        k[0, h, :half] = ints
        k[0, h, half:] = -ints
        for b0 in range(0, S, O.BK):
            k[0, h, b0:b0 + O.BK] *= 2.0 ** -(3 + (b0 // O.BK) % 4)
    return q.astype(np.float16), k.astype(np.float16)


@pytest.mark.parametrize("causal,tile,kv_map", [(False, 64, None), (True, 64, None),
                                                (True, 1, None), (False, 100, [1, 0, 1, 0]),
                                                (True, 512, None)])
def test_pv8_online_machinery_without_weight_rounding_is_exact_attention(causal, tile, kv_map):
    """With p unrounded and V on an exact per-channel E4M3 grid, the online
    algorithm must give exact attention for any tile size (tiling, rescaling,
    masking and the head map are pinned; only the weight rounding is off)."""
    rng = np.random.default_rng(61 + tile)
    S, D, Hq, Hkv = 512, 32, 4, 2
    q, k = _int8_lossless(rng, S, D, Hq, Hkv)
    v = _lossless_v(rng, Hkv, S, D)
    qz = O.quantize_qk(q, k)
    codes, vs = O.quant_v_fp8(v)
    assert np.array_equal(_torch_decode(codes) * vs[:, :, None, :].astype(np.float64), v.astype(np.float64))
    o_exact, lse_exact = O.attention(q, k, v, causal=causal, kv_map=kv_map, with_lse=True)
    o5, lse5 = O.pv8_attention(qz, codes, vs, causal=causal, kv_map=kv_map, tile=tile,
                               p_quant=False, with_lse=True)
    np.testing.assert_allclose(o5, o_exact, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse5, lse_exact, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_pv8_equal_scores_give_the_mean_of_v(causal):
    """Q = 0: every score is 0, every weight is 1 and 448 * 1 is an E4M3 value,
    so O is the (prefix) mean of the 8-bit V exactly."""
    rng = np.random.default_rng(71)
    S, D = 200, 64
    q = np.zeros((1, 2, S, D), np.float16)
    k = rng.standard_normal((1, 1, S, D)).astype(np.float16)
    v = rng.standard_normal((1, 1, S, D)).astype(np.float16)
    qz = O.quantize_qk(q, k)
    codes, vs = O.quant_v_fp8(v)
    vq = _torch_decode(codes) * vs[:, :, None, :].astype(np.float64)
    o5 = O.pv8_attention(qz, codes, vs, causal=causal)
    if causal:
        ref = np.cumsum(vq[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    else:
        ref = np.broadcast_to(vq[0, 0].mean(axis=0), (S, D))
    for h in range(2):
        np.testing.assert_allclose(o5[0, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_pv8_weight_rounding_error_bound(causal):
    """Rounding each weight to E4M3 moves it by at most 2^-4 of itself (normal
    range) or 2^-10 / 448 (subnormal range), so with l from unrounded weights
    |O_rounded - O_unrounded| <= (2^-4 + n 2^-10 / 448) max|V'| for n visible keys."""
    rng = np.random.default_rng(81)
    S, D = 256, 64
    q = (rng.standard_normal((1, 2, S, D)) * 2).astype(np.float16)
    k = rng.standard_normal((1, 1, S, D)).astype(np.float16)
    v = rng.standard_normal((1, 1, S, D)).astype(np.float16)
    qz = O.quantize_qk(q, k)
    codes, vs = O.quant_v_fp8(v)
    vmax = np.abs(_torch_decode(codes) * vs[:, :, None, :]).max()
    o_r = O.pv8_attention(qz, codes, vs, causal=causal, p_quant=True)
    o_u = O.pv8_attention(qz, codes, vs, causal=causal, p_quant=False)
    n = (np.arange(S) + 1) if causal else np.full(S, S)
    bound = (2.0 ** -4 + n * 2.0 ** -10 / 448) * vmax
    assert np.all(np.abs(o_r - o_u).max(axis=-1) <= bound[None, None, :] * (1 + 1e-9))
    assert np.abs(o_r - o_u).max() > 0          # the rounding does act


# --------------------------------------------------------------------------
# O5's rounding point, pinned by a hand computation
# --------------------------------------------------------------------------
def _e4m3_grid():
    """Every non-negative finite E4M3 value from the format's definition
    (exponent bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, exponent field
    15 with mantissa 7 the NaN, so 448 is the largest value), exactly."""
    vals = [Fraction(m, 8) * Fraction(1, 64) for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if not (e == 15 and m == 7):
                vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return sorted(vals)


_GRID = _e4m3_grid()


def _round_and_tie(x: Decimal):
    """Nearest E4M3 value of 0 < x <= 448 (exact; no tie may occur here), the
    larger of the grid gaps on either side of it (the most a rounding to the
    other side can move it) and x's relative distance from the nearest
    half-way point between two neighbouring grid values."""
    xf = Fraction(x)
    hi = next(i for i, g in enumerate(_GRID) if g >= xf)
    if xf == _GRID[hi]:                      # on the grid: the half-way points on either side
        gaps = [_GRID[hi] - _GRID[hi - 1]] + ([_GRID[hi + 1] - _GRID[hi]] if hi + 1 < len(_GRID) else [])
        return xf, max(gaps), min(gaps) / 2 / xf
    below, above = _GRID[hi - 1], _GRID[hi]
    assert abs((xf - below) - (above - xf)) > Fraction(1, 10 ** 30) * xf, "a tie"
    nearest = below if xf - below < above - xf else above
    return nearest, above - below, abs(xf - (below + above) / 2) / xf


def _hand_pv8(a, vq, tile, tie_rel=None):
    """O of one query row in closed form, 50-digit decimals: scores a_j ln2/8
    (so exp(s_j - m) = 2^((a_j - m)/8)); key j is weighted by
    E4M3(448 2^((a_j - M_t)/8)) / 448 * 2^((M_t - M)/8), where M_t is the
    maximum of the scores up to the end of j's tile of `tile` keys and M the
    row maximum; l = sum_j 2^((a_j - M)/8) (unrounded).  Also the tie slack of
    the weights whose 448 p lies within tie_rel of a half-way point."""
    getcontext().prec = 50
    two = Decimal(2)
    n = len(a)
    M = max(a)
    l = sum(two ** (Decimal(int(x - M)) / 8) for x in a)
    acc = [Decimal(0)] * vq.shape[1]
    slack = Decimal(0)
    rel = []
    for j in range(n):
        Mt = max(a[:min(n, (j // tile + 1) * tile)])
        x = 448 * two ** (Decimal(int(a[j] - Mt)) / 8)
        r, step, d = _round_and_tie(x)
        carry = two ** (Decimal(int(Mt - M)) / 8)
        w = Decimal(r.numerator) / Decimal(r.denominator) / 448 * carry
        for c in range(vq.shape[1]):
            acc[c] += w * Decimal(float(vq[j, c]))
        rel.append(d)
        if tie_rel is not None and d <= Fraction(tie_rel):
            slack += Decimal(step.numerator) / Decimal(step.denominator) / 448 * carry * \
                Decimal(float(np.abs(vq[j]).max()))
    return np.array([float(x / l) for x in acc]), float(slack / l), rel


def _two_tile_case():
    """One row over 128 keys (two 64-key tiles): keys 0-31 peak at 40, keys
    32-63 at 60 and keys 64-127 at 75, so the running maximum rises inside the
    first 64 keys (at a 32-key boundary) and again in the second tile, by
    amounts that are not multiples of 8 (the rescale factors are not powers of
    two, which rounding would commute with)."""
    rng = np.random.default_rng(2025)
    S, D = 128, 16
    a = np.concatenate([rng.integers(0, 41, 32), rng.integers(10, 61, 32), rng.integers(30, 76, 64)])
    a[5], a[40], a[100] = 40, 60, 75
    q_i8 = np.zeros((1, 1, S, D), np.int8)
    q_i8[..., 0] = 1
    k_i8 = np.zeros((1, 1, S, D), np.int8)
    k_i8[0, 0, :, 0] = a
    qz = dict(q_i8=q_i8, q_scale=np.ones((1, 1, 1), np.float32), k_i8=k_i8,
              k_scale=np.ones((1, 1, 2), np.float32))
    finite = _finite_codes()
    mag = finite[(O.e4m3_decode(finite) >= 0.25) & (O.e4m3_decode(finite) <= 4)]
    codes = rng.choice(mag, (1, 1, S, D)).astype(np.uint8)
    vq = _torch_decode(codes)[0, 0]
    return qz, codes, np.ones((1, 1, D), np.float32), a, vq


def test_pv8_rounds_each_weight_against_the_running_maximum_of_its_64_key_tile():
    """R20 pinned: O5 equals the closed form with 64-key tiles (the running
    maximum at the end of each key's tile), and that value differs from both
    alternative readings -- 32-key tiles, and rounding against the final row
    maximum -- by far more than the comparison's tolerance, so O5 computed
    under either of them fails this test.  O5 with tile = 32 and tile = 128
    (one tile: the final maximum) matches the closed form of that reading
    too, which checks the closed form itself."""
    qz, codes, vs, a, vq = _two_tile_case()
    sm = float(np.log(2.0) / 8)
    hand = {t: _hand_pv8(list(a), vq, t)[0] for t in (64, 32, 128)}
    for t in (64, 32, 128):
        o5 = O.pv8_attention(qz, codes, vs, sm_scale=sm, tile=t, rows=np.array([0], np.int32))[0, 0, 0]
        np.testing.assert_allclose(o5, hand[t], rtol=0, atol=1e-12)
    assert np.abs(hand[64] - hand[32]).max() > 1e-4
    assert np.abs(hand[64] - hand[128]).max() > 1e-4
    o5 = O.pv8_attention(qz, codes, vs, sm_scale=sm, rows=np.array([0], np.int32))[0, 0, 0]   # default tile
    np.testing.assert_allclose(o5, hand[64], rtol=0, atol=1e-12)


def test_pv8_tie_slack_against_the_hand_computation():
    """The per-row tie slack: 0 at tie_rel = 0; with tie_rel just above the
    k-th smallest relative distance of a weight from an E4M3 half-way point
    it sums exactly the k weights that close (one grid step each, carried to
    the final maximum, times the row's largest |V'|, over l)."""
    qz, codes, vs, a, vq = _two_tile_case()
    sm = float(np.log(2.0) / 8)
    row = np.array([0], np.int32)
    _, s0 = O.pv8_attention(qz, codes, vs, sm_scale=sm, rows=row, tie_rel=0.0)
    assert s0[0, 0, 0] == 0.0
    _, _, rel = _hand_pv8(list(a), vq, 64)
    order = sorted(float(r) for r in rel)
    for k in (1, 5, 20, 128):
        tie_rel = order[k - 1] * (1 + 1e-9) if k < 128 else 1.0
        _, hand_slack, _ = _hand_pv8(list(a), vq, 64, tie_rel=tie_rel)
        _, sl = O.pv8_attention(qz, codes, vs, sm_scale=sm, rows=row, tie_rel=tie_rel)
        np.testing.assert_allclose(sl[0, 0, 0], hand_slack, rtol=1e-12, atol=0)
    assert hand_slack > 0


# --------------------------------------------------------------------------
# the pages' accuracy claims, on the workloads' value distributions
# --------------------------------------------------------------------------
def _cos_rel_l1(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    return a @ b / (np.linalg.norm(a) * np.linalg.norm(b)), np.abs(a - b).sum() / np.abs(b).sum()


@pytest.mark.parametrize("name", ["tiny_mha", "llm_prefill_gqa"])
def test_int8_qk_is_more_accurate_than_fp8_and_8bit_pv(name):
    from bit_quantized_exact_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS[name]
    if w.seq > 1024 or w.batch > 1:
        w = w.scaled(batch=1, heads_q=min(w.heads_q, 8), heads_kv=min(w.heads_kv, 2), seq=1024)
    q, k, v = make_qkv(w)
    rows = None if w.seq <= 256 else np.arange(0, w.seq, 7)
    exact = O.attention(q, k, v, causal=w.causal, rows=rows)
    qz = O.quantize_qk(q, k)
    i8 = _cos_rel_l1(O.quant_attention(qz, v, causal=w.causal, rows=rows), exact)
    f8 = _cos_rel_l1(O.quant_attention_fp8(O.quantize_qk_fp8(q, k), v, causal=w.causal, rows=rows), exact)
    codes, vs = O.quant_v_fp8(v)
    pv = _cos_rel_l1(O.pv8_attention(qz, codes, vs, causal=w.causal, rows=rows), exact)
    assert i8[1] < f8[1] / 2 and i8[1] < pv[1] / 2, (i8, f8, pv)
    assert i8[0] > f8[0] and i8[0] > pv[0]
