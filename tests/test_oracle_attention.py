"""Pins of the exact-attention oracle (O1) against what the pages and mathematics fix.

Sources: "注意力即一切：从 MHA 到 GQA" §2.2 (scores, softmax of score/sqrt(d_k),
weights sum to one, weighted sum of V), §2.3 (causal: future keys get weight 0),
§4.1/§5.1 (MQA/GQA: a group of query heads shares one K/V head; g = h is MHA);
SageAttention article, 技术方案: softmax(QK^T) = softmax(Q(K - mean K)^T).

None of these tests re-types the oracle's formula: each checks it against an
independent evaluation (40-digit decimal arithmetic, torch's CPU
scaled_dot_product_attention in float64, a closed form) or an invariant.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle import oracle as O


def _f16(rng, shape, scale=1.0, offset=None):
    x = rng.standard_normal(shape) * scale
    if offset is not None:
        x = x + offset
    return x.astype(np.float16)


# --------------------------------------------------------------------------
# fp16 decoding / rounding helpers
# --------------------------------------------------------------------------
def test_half_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.half_to_double(bits.view(np.float16))
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_round_to_half_matches_numpy():
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        rng.random(20000),                         # weights in [0, 1)
        rng.random(2000) * 1e-5,                   # subnormal range
        np.ldexp(rng.integers(1, 2048, 2000) + 0.5, -24),   # exact ties (subnormal)
        np.ldexp(rng.integers(1024, 2048, 2000) + 0.5, -11),  # exact ties (normal)
        [1.0, 0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 65504.0],
    ])
    got = np.array([O.round_to_half(x) for x in xs])
    ref = xs.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# brute force at 40 digits, seq <= 16
# --------------------------------------------------------------------------
def _decimal_attention(q, k, v, causal, kv_map, sm):
    getcontext().prec = 40
    B, Hq, S, D = q.shape
    out = np.zeros(q.shape, dtype=np.float64)
    smd = Decimal(float(sm))
    for b in range(B):
        for h in range(Hq):
            kh = kv_map[h]
            for i in range(S):
                js = [j for j in range(S) if (not causal or j <= i)]
                s = []
                for j in js:
                    dot = sum(Decimal(float(q[b, h, i, c])) * Decimal(float(k[b, kh, j, c]))
                              for c in range(D))
                    s.append(dot * smd)
                m = max(s)
                p = [(x - m).exp() for x in s]
                l = sum(p)
                for c in range(D):
                    num = sum(pj * Decimal(float(v[b, kh, j, c])) for pj, j in zip(p, js))
                    out[b, h, i, c] = float(num / l)
    return out


@pytest.mark.parametrize("S,D,Hq,Hkv,causal", [
    (1, 4, 1, 1, False), (2, 8, 2, 1, True), (5, 8, 2, 2, False),
    (9, 16, 4, 2, True), (16, 8, 3, 1, False), (16, 16, 2, 2, True)])
def test_bruteforce_decimal(S, D, Hq, Hkv, causal):
    rng = np.random.default_rng(100 + S * 7 + D)
    q = _f16(rng, (1, Hq, S, D), 1.5)
    k = _f16(rng, (1, Hkv, S, D), 1.0, offset=rng.standard_normal((1, Hkv, 1, D)) * 2)
    v = _f16(rng, (1, Hkv, S, D))
    kv_map = np.arange(Hq) // (Hq // Hkv)
    sm = 1.0 / math.sqrt(D)
    got = O.attention(q, k, v, causal=causal)
    ref = _decimal_attention(q, k, v, causal, kv_map, sm)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# torch CPU scaled_dot_product_attention in float64 (the routine the method
# replaces), seq <= 512
# --------------------------------------------------------------------------
def _sdpa(q, k, v, causal, kv_map, scale=None):
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))[:, kv_map]
    vt = torch.from_numpy(v.astype(np.float64))[:, kv_map]
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("S,D,Hq,Hkv,causal", [
    (1, 64, 2, 2, False), (7, 64, 4, 1, True), (64, 128, 4, 2, True),
    (129, 64, 2, 2, False), (300, 128, 8, 2, True), (512, 64, 2, 1, False)])
def test_against_torch_sdpa_f64(S, D, Hq, Hkv, causal):
    rng = np.random.default_rng(S * 31 + D)
    q = _f16(rng, (2, Hq, S, D))
    k = _f16(rng, (2, Hkv, S, D), 1.0, offset=rng.standard_normal((2, Hkv, 1, D)) * 3)
    v = _f16(rng, (2, Hkv, S, D))
    kv_map = np.arange(Hq) // (Hq // Hkv)
    got = O.attention(q, k, v, causal=causal)
    ref = _sdpa(q, k, v, causal, kv_map)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_explicit_noncontiguous_map_against_sdpa():
    rng = np.random.default_rng(5)
    S, D, Hq, Hkv = 96, 64, 6, 3
    q = _f16(rng, (1, Hq, S, D))
    k = _f16(rng, (1, Hkv, S, D))
    v = _f16(rng, (1, Hkv, S, D))
    kv_map = np.array([2, 0, 1, 1, 0, 2], dtype=np.int32)
    got = O.attention(q, k, v, causal=True, kv_map=kv_map)
    np.testing.assert_allclose(got, _sdpa(q, k, v, True, kv_map), rtol=0, atol=1e-12)


def test_custom_scale_against_sdpa():
    rng = np.random.default_rng(6)
    q = _f16(rng, (1, 2, 40, 64))
    k = _f16(rng, (1, 2, 40, 64))
    v = _f16(rng, (1, 2, 40, 64))
    got = O.attention(q, k, v, sm_scale=0.3)
    np.testing.assert_allclose(got, _sdpa(q, k, v, False, [0, 1], scale=0.3), rtol=0, atol=1e-12)


def test_lse_against_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(8)
    S, D = 77, 64
    q = _f16(rng, (1, 2, S, D))
    k = _f16(rng, (1, 2, S, D))
    v = _f16(rng, (1, 2, S, D))
    for causal in (False, True):
        _, lse = O.attention(q, k, v, causal=causal, with_lse=True)
        s = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64)) / 8.0
        if causal:
            s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        np.testing.assert_allclose(lse, logsumexp(s, axis=-1), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_constant_v_gives_the_constant():
    rng = np.random.default_rng(9)
    q = _f16(rng, (1, 2, 50, 64), 3.0)
    k = _f16(rng, (1, 2, 50, 64), 3.0)
    v = np.full((1, 2, 50, 64), 0.7109375, dtype=np.float16)  # exact in fp16
    for causal in (False, True):
        out = O.attention(q, k, v, causal=causal)
        np.testing.assert_allclose(out, 0.7109375, rtol=0, atol=1e-15)


def test_weights_sum_to_one():
    rng = np.random.default_rng(10)
    q = _f16(rng, (1, 3, 33, 64), 2.0)
    k = _f16(rng, (1, 3, 33, 64), 2.0)
    ones = np.ones((1, 3, 33, 64), dtype=np.float16)
    np.testing.assert_allclose(O.attention(q, k, ones), 1.0, rtol=0, atol=1e-14)


def test_causal_row0_and_single_key():
    rng = np.random.default_rng(11)
    q = _f16(rng, (2, 2, 20, 64))
    k = _f16(rng, (2, 2, 20, 64))
    v = _f16(rng, (2, 2, 20, 64))
    out = O.attention(q, k, v, causal=True)
    assert np.array_equal(out[:, :, 0], v[:, :, 0].astype(np.float64))
    one = O.attention(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    assert np.array_equal(one[:, :, 0], v[:, :, 0].astype(np.float64))


def test_two_keys_closed_form():
    # q . k0 = 1, q . k1 = 0 with D = 4, scale 1/2: weights e^(1/2) and 1.
    q = np.array([1, 0, 0, 0], np.float16).reshape(1, 1, 1, 4)
    q = np.repeat(q, 2, axis=2)
    k = np.array([[1, 0, 0, 0], [0, 1, 0, 0]], np.float16).reshape(1, 1, 2, 4)
    v = np.array([[1, 2, 3, 4], [-4, 0.5, 0, 8]], np.float16).reshape(1, 1, 2, 4)
    out = O.attention(q, k, v)
    w0 = math.exp(0.5) / (math.exp(0.5) + 1.0)
    expect = w0 * v[0, 0, 0].astype(np.float64) + (1 - w0) * v[0, 0, 1].astype(np.float64)
    np.testing.assert_allclose(out[0, 0, 0], expect, rtol=0, atol=1e-15)
    # causal row 0 only sees key 0
    outc = O.attention(q, k, v, causal=True)
    np.testing.assert_array_equal(outc[0, 0, 0], v[0, 0, 0].astype(np.float64))
    np.testing.assert_allclose(outc[0, 0, 1], expect, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_channel_shift_invariance(causal):
    """softmax(QK^T) = softmax(Q(K - c)^T) for a per-channel constant c (SageAttention, 技术方案)."""
    rng = np.random.default_rng(12)
    S, D = 70, 64
    q = (rng.integers(-64, 64, (1, 2, S, D)) / 32.0).astype(np.float16)
    base = (rng.integers(-64, 64, (1, 2, S, D)) / 32.0).astype(np.float16)
    c = (rng.integers(-256, 256, (1, 2, 1, D)) / 32.0)
    k_shift = (base.astype(np.float64) + c).astype(np.float16)   # exact: multiples of 1/32
    assert np.array_equal(k_shift.astype(np.float64), base.astype(np.float64) + c)
    v = _f16(rng, (1, 2, S, D))
    a = O.attention(q, base, v, causal=causal)
    b = O.attention(q, k_shift, v, causal=causal)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(13)
    S, D, Hq, Hkv = 60, 64, 8, 2
    q = _f16(rng, (1, Hq, S, D))
    k = _f16(rng, (1, Hkv, S, D))
    v = _f16(rng, (1, Hkv, S, D))
    g = O.attention(q, k, v, causal=True)
    rep_k = np.repeat(k, Hq // Hkv, axis=1)
    rep_v = np.repeat(v, Hq // Hkv, axis=1)
    m = O.attention(q, rep_k, rep_v, causal=True)
    assert np.array_equal(g, m)
    # g = 1 (MQA) equals MHA on the broadcast head
    mq = O.attention(q, k[:, :1], v[:, :1], causal=True)
    mm = O.attention(q, np.repeat(k[:, :1], Hq, 1), np.repeat(v[:, :1], Hq, 1), causal=True)
    assert np.array_equal(mq, mm)


def test_kv_head_change_only_affects_its_group():
    rng = np.random.default_rng(14)
    S, D, Hq, Hkv = 40, 64, 6, 3
    q = _f16(rng, (1, Hq, S, D))
    k = _f16(rng, (1, Hkv, S, D))
    v = _f16(rng, (1, Hkv, S, D))
    kv_map = np.array([1, 1, 0, 2, 0, 2], np.int32)
    a = O.attention(q, k, v, kv_map=kv_map)
    k2 = k.copy()
    k2[0, 2] = _f16(rng, (S, D))
    b = O.attention(q, k2, v, kv_map=kv_map)
    changed = [h for h in range(Hq) if not np.array_equal(a[0, h], b[0, h])]
    assert changed == [3, 5]


def test_causal_future_keys_have_no_weight():
    rng = np.random.default_rng(15)
    S, D = 48, 64
    q = _f16(rng, (1, 2, S, D))
    k = _f16(rng, (1, 2, S, D))
    v = _f16(rng, (1, 2, S, D))
    a = O.attention(q, k, v, causal=True)
    t = 30
    k2, v2 = k.copy(), v.copy()
    k2[:, :, t + 1:] = _f16(rng, (1, 2, S - t - 1, D), 5.0)
    v2[:, :, t + 1:] = _f16(rng, (1, 2, S - t - 1, D), 5.0)
    b = O.attention(q, k2, v2, causal=True)
    assert np.array_equal(a[:, :, :t + 1], b[:, :, :t + 1])
    assert not np.array_equal(a[:, :, t + 1:], b[:, :, t + 1:])


def test_row_subset_matches_full():
    rng = np.random.default_rng(16)
    q = _f16(rng, (2, 4, 130, 64))
    k = _f16(rng, (2, 2, 130, 64))
    v = _f16(rng, (2, 2, 130, 64))
    full = O.attention(q, k, v, causal=True)
    rows = np.array([0, 5, 127, 128, 129])
    sub = O.attention(q, k, v, causal=True, rows=rows)
    assert np.array_equal(sub, full[:, :, rows])
