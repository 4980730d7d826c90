"""Pins of the smoothing / quantisation model (O2-O4) of the oracle.

Source: SageAttention article ("又快又准，即插即用！清华8比特量化Attention…"),
section 技术方案: K <- K - mean(K); Q and K quantised to INT8 per
FlashAttention-sized block; QK^T as an INT8 product with INT32 accumulation;
P and V kept in FP16.  The pages print no scale formula or rounding rule; the
readings (symmetric absmax, 127/a in fp32, round-half-even, saturation at
+-127, fp64 mean rounded to fp32) are pinned here against exact rational
arithmetic and invariants, not against a re-typing of the code.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O


def _f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


# --------------------------------------------------------------------------
# O2: channel mean over tokens
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 3, 64, 100, 128, 257])
def test_k_mean_against_exact_fraction(S):
    rng = np.random.default_rng(S)
    D = 16
    k = _f16(rng, (2, 2, S, D), 4.0)
    k = (k.astype(np.float32) + rng.standard_normal((2, 2, 1, D)).astype(np.float32) * 8).astype(np.float16)
    mu = O.k_mean(k)
    for b in range(2):
        for h in range(2):
            for c in range(D):
                exact = sum(Fraction(float(x)) for x in k[b, h, :, c]) / S
                got = Fraction(float(mu[b, h, c]))
                # correctly rounded to fp32: within half an ulp of the exact mean
                e = float(exact)
                ulp = float(np.spacing(np.float32(abs(e)))) if e != 0 else 2.0 ** -149
                assert abs(got - exact) <= Fraction(ulp) / 2
                if S & (S - 1) == 0:   # S a power of two: a single rounding, exact match
                    assert mu[b, h, c] == np.float32(float(exact))


def test_k_mean_is_over_tokens_not_channels():
    # K[j, c] = c for every token j: the per-channel mean is c, the per-token mean would be (D-1)/2
    D, S = 8, 32
    k = np.broadcast_to(np.arange(D, dtype=np.float16), (1, 1, S, D)).copy()
    mu = O.k_mean(k)
    assert np.array_equal(mu[0, 0], np.arange(D, dtype=np.float32))


def test_k_mean_rejects_inexact_sums():
    k = np.full((1, 1, 16384, 4), 60000.0, dtype=np.float16)   # sum |K| ~ 9.8e8 > 2^29
    with pytest.raises(RuntimeError):
        O.k_mean(k)


def test_smoothed_k_has_zero_channel_mean():
    rng = np.random.default_rng(3)
    k = _f16(rng, (1, 2, 256, 64), 1.0)
    k = (k.astype(np.float32) + np.float32(5.0) * rng.standard_normal((1, 2, 1, 64)).astype(np.float32)).astype(np.float16)
    mu = O.k_mean(k)
    ks = O.smooth_k(k, mu)
    assert np.abs(ks.astype(np.float64).mean(axis=2)).max() < 1e-5
    # the shift is the same for every token: ks[j] - ks[0] equals K[j] - K[0] exactly here
    diff = ks - ks[:, :, :1]
    ref = k.astype(np.float32) - k[:, :, :1].astype(np.float32)
    np.testing.assert_allclose(diff, ref, rtol=0, atol=1e-5)


# --------------------------------------------------------------------------
# O3: block quantisation
# --------------------------------------------------------------------------
def _blocks(x, block):
    S = x.shape[-2]
    return [(b0, min(S, b0 + block)) for b0 in range(0, S, block)]


@pytest.mark.parametrize("S,block", [(128, 128), (200, 64), (7, 64), (129, 128)])
def test_quant_invariants(S, block):
    rng = np.random.default_rng(S + block)
    x = (rng.standard_normal((3, S, 32)) * rng.uniform(0.01, 50, (3, 1, 1))).astype(np.float32)
    q, sc = O.quant_blocks(x, block)
    assert sc.shape == (3, (S + block - 1) // block)
    assert np.abs(q.astype(np.int32)).max() <= 127
    for m in range(3):
        for bi, (r0, r1) in enumerate(_blocks(x, block)):
            xb = x[m, r0:r1]
            qb = q[m, r0:r1].astype(np.int64)
            a = np.abs(xb).max()
            # the absmax element maps to +-127
            i = np.unravel_index(np.abs(xb).argmax(), xb.shape)
            assert abs(qb[i]) == 127 and np.sign(qb[i]) == np.sign(xb[i])
            # delta = a / 127 rounded to fp32
            d = sc[m, bi]
            assert Fraction(float(d)) == Fraction(float(a)) / 127 or \
                abs(Fraction(float(d)) - Fraction(float(a)) / 127) <= Fraction(float(np.spacing(d))) / 2
            # reconstruction error: at most half a step, plus a few fp32 roundings
            err = np.abs(xb.astype(np.float64) - qb * float(d))
            assert err.max() <= float(d) * (0.5 + 2.0 ** -15)


def test_quant_rounds_to_nearest_of_exact_ratio():
    """q is the integer nearest to x*127/a (exact rational), away from near-ties."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((4, 64, 16)) * 3).astype(np.float32)
    q, _ = O.quant_blocks(x, 64)
    for m in range(4):
        a = Fraction(float(np.abs(x[m]).max()))
        for (j, c), xv in np.ndenumerate(x[m]):
            t = Fraction(float(xv)) * 127 / a
            frac = t - math.floor(t)
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 16):
                continue   # a near-tie: decided by the fp32 product, not pinned here
            nearest = math.floor(t + Fraction(1, 2))
            assert q[m, j, c] == nearest


def test_quant_exact_ties_round_half_even():
    # a = 127 -> r = 1 exactly; x = k + 0.5 are exact ties
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]], np.float32)
    q, sc = O.quant_blocks(x.reshape(1, 1, 8), 1)
    assert q.ravel().tolist() == [127, 0, 2, 2, 0, -2, -2, 4]
    assert sc.ravel()[0] == np.float32(1.0)


def test_quant_zero_block_and_symmetry():
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((2, 192, 16))).astype(np.float32)
    x[0, 64:128] = 0.0
    q, sc = O.quant_blocks(x, 64)
    assert sc[0, 1] == 0.0 and not q[0, 64:128].any()
    qn, scn = O.quant_blocks(-x, 64)
    assert np.array_equal(qn, -q) and np.array_equal(scn, sc)


def test_quant_scale_invariance_power_of_two():
    # multiplying a block by 2^k scales delta by 2^k and leaves q unchanged
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((1, 128, 64))).astype(np.float32)
    q1, s1 = O.quant_blocks(x, 64)
    q2, s2 = O.quant_blocks(x * np.float32(8.0), 64)
    assert np.array_equal(q1, q2) and np.array_equal(s2, s1 * 8)


# --------------------------------------------------------------------------
# integer scores
# --------------------------------------------------------------------------
def test_scores_against_python_int_bruteforce():
    rng = np.random.default_rng(31)
    S, D, Hq, Hkv = 9, 16, 4, 2
    qi = rng.integers(-127, 128, (1, Hq, S, D)).astype(np.int8)
    ki = rng.integers(-127, 128, (1, Hkv, S, D)).astype(np.int8)
    kv_map = [1, 0, 0, 1]
    for causal in (False, True):
        s = O.scores_i32(qi, ki, causal=causal, kv_map=kv_map, fill=-7)
        for h in range(Hq):
            for i in range(S):
                for j in range(S):
                    if causal and j > i:
                        assert s[0, h, i, j] == -7
                    else:
                        ref = sum(int(qi[0, h, i, c]) * int(ki[0, kv_map[h], j, c]) for c in range(D))
                        assert s[0, h, i, j] == ref


def test_scores_extreme_values_and_int64_matmul():
    rng = np.random.default_rng(32)
    S, D = 300, 128
    qi = rng.choice(np.array([-127, 127], np.int8), (1, 2, S, D))
    ki = rng.integers(-127, 128, (1, 2, S, D)).astype(np.int8)
    ki[0, 0, 5] = qi[0, 0, 3]          # a score of D*127^2
    s = O.scores_i32(qi, ki)
    ref = np.matmul(qi.astype(np.int64), np.swapaxes(ki.astype(np.int64), -1, -2))
    assert np.array_equal(s, ref)
    assert s[0, 0, 3, 5] == D * 127 * 127


# --------------------------------------------------------------------------
# O4 quantised attention: the lossless grid pins the dequantisation factor
# --------------------------------------------------------------------------
def _lossless_inputs(rng, S, D, Hq, Hkv, bq, bk):
    """Q, K whose blocks are exact integer multiples of a power-of-two step with
    a +-127*step element in every block, and K channel sums of exactly zero."""
    q = np.zeros((1, Hq, S, D))
    for h in range(Hq):
        for b0 in range(0, S, bq):
            step = 2.0 ** -(3 + (b0 // bq + h) % 3)
            n = min(bq, S - b0)
            blk = rng.integers(-127, 128, (n, D)).astype(np.float64)
            blk[0, 0] = 127
            q[0, h, b0:b0 + n] = blk * step
    assert S % (2 * bk) == 0
    k = np.zeros((1, Hkv, S, D))
    half = S // 2
    for h in range(Hkv):
        ints = rng.integers(-127, 128, (half, D)).astype(np.float64)
        ints[::bk, 0] = -127                     # an extreme element in every block
        k[0, h, :half] = ints
        k[0, h, half:] = -ints                   # channel sums are exactly zero
        for b0 in range(0, S, bk):
            k[0, h, b0:b0 + bk] *= 2.0 ** -(2 + (b0 // bk) % 4)
    # zero means need equal steps for rows j and j+S/2: the block pattern repeats every 4 blocks
    assert (half // bk) % 4 == 0
    return q.astype(np.float16), k.astype(np.float16)


@pytest.mark.parametrize("causal", [False, True])
def test_lossless_grid_dequantisation(causal):
    rng = np.random.default_rng(41)
    S, D, Hq, Hkv = 512, 64, 4, 2
    q, k = _lossless_inputs(rng, S, D, Hq, Hkv, O.BQ, O.BK)
    v = _f16(rng, (1, Hkv, S, D))
    qz = O.quantize_qk(q, k)
    assert not qz["k_mean"].any()               # mu = 0 exactly
    # quantisation is exact: int8 * delta reproduces the inputs
    dq = np.repeat(qz["q_scale"], O.BQ, axis=-1)[..., :S, None]
    dk = np.repeat(qz["k_scale"], O.BK, axis=-1)[..., :S, None]
    assert np.array_equal(qz["q_i8"] * dq.astype(np.float64), q.astype(np.float64))
    assert np.array_equal(qz["k_i8"] * dk.astype(np.float64), k.astype(np.float64))
    # lse does not see the fp16 rounding of P when l uses unrounded weights: exact match
    o_exact, lse_exact = O.attention(q, k, v, causal=causal, with_lse=True)
    o_q, lse_q = O.quant_attention(qz, v, causal=causal, with_lse=True)
    np.testing.assert_allclose(lse_q, lse_exact, rtol=0, atol=1e-12)
    # the output differs from exact only by the fp16 rounding of the weights
    np.testing.assert_allclose(o_q, o_exact, rtol=0, atol=2e-3)


def test_fp16_weight_rounding_is_what_separates_o4_from_o1():
    rng = np.random.default_rng(42)
    S, D = 512, 64
    q, k = _lossless_inputs(rng, S, D, 2, 1, O.BQ, O.BK)
    v = np.ones((1, 1, S, D), np.float16)
    qz = O.quantize_qk(q, k)
    # with l summed from the rounded weights, constant V is reproduced exactly
    o = O.quant_attention(qz, v, l_from_rounded=True)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)


def test_block_sizes_exported():
    assert (O.BQ, O.BK) == (128, 64)


def _cos_rel_l1(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    cos = a @ b / (np.linalg.norm(a) * np.linalg.norm(b))
    return cos, np.abs(a - b).sum() / np.abs(b).sum()


@pytest.mark.parametrize("name", ["tiny_mha", "llm_prefill_gqa", "batched_mqa"])
def test_quantised_model_meets_accuracy_bar_on_workload_distributions(name):
    """The readings (per-channel mean over tokens, BQ=128/BK=64 blocks) meet
    cos >= 0.999 and rel-L1 <= 0.02 against exact attention on the workloads'
    value distributions (reduced sequence length for the large ones)."""
    from bit_quantized_exact_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS[name]
    if w.seq > 1024 or w.batch > 1:
        w = w.scaled(batch=1, heads_q=min(w.heads_q, 8), heads_kv=min(w.heads_kv, 2), seq=1024)
    q, k, v = make_qkv(w)
    qz = O.quantize_qk(q, k)
    rows = None if w.seq <= 256 else np.arange(0, w.seq, 7)
    exact = O.attention(q, k, v, causal=w.causal, rows=rows)
    approx = O.quant_attention(qz, v, causal=w.causal, rows=rows)
    cos, rl1 = _cos_rel_l1(approx, exact)
    assert cos >= 0.999 and rl1 <= 0.02, (cos, rl1)
