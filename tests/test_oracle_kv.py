"""Pins of the oracle's KV-cache (decode) functions: Sq queries over Sk >= Sq
cached keys ("注意力即一切：从 MHA 到 GQA" §3.4: the keys and values of
all earlier tokens are cached and the current token's queries attend over
them).  The queries are the last Sq positions, so the causal mask is aligned
bottom-right.  Pinned by: equality with the square functions when Sq = Sk
(written separately), decode rows = the last rows of a full causal prefill
(the alignment), and the lossless-grid case of the quantised model.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _f16(rng, shape, scale=1.0, offset=None):
    x = rng.standard_normal(shape) * scale
    if offset is not None:
        x = x + offset
    return x.astype(np.float16)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kv_map", [None, [1, 0, 1]])
def test_square_case_equals_square_oracle(causal, kv_map):
    rng = np.random.default_rng(1)
    Hq = 4 if kv_map is None else 3
    q = _f16(rng, (2, Hq, 70, 32))
    k = _f16(rng, (2, 2, 70, 32), offset=rng.standard_normal(32) * 2)
    v = _f16(rng, (2, 2, 70, 32))
    a, la = O.attention_kv(q, k, v, causal=causal, kv_map=kv_map, with_lse=True)
    b, lb = O.attention(q, k, v, causal=causal, kv_map=kv_map, with_lse=True)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 300), (3, 300), (16, 129), (32, 64), (7, 7)])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_rows_are_the_last_rows_of_prefill(Sq, Sk, causal):
    """Bottom-right alignment: the Sq decode queries are positions Sk-Sq..Sk-1."""
    rng = np.random.default_rng(Sq * 1000 + Sk)
    q_full = _f16(rng, (1, 4, Sk, 64))
    k = _f16(rng, (1, 2, Sk, 64), offset=rng.standard_normal(64))
    v = _f16(rng, (1, 2, Sk, 64))
    dec = O.attention_kv(q_full[:, :, Sk - Sq:], k, v, causal=causal)
    ref = O.attention(q_full, k, v, causal=causal, rows=np.arange(Sk - Sq, Sk))
    np.testing.assert_allclose(dec, ref, rtol=0, atol=1e-13)


def test_single_query_causal_sees_every_cached_key():
    """One decode query under the causal mask attends over all Sk keys: equal
    to the non-causal result, and with equal scores to the mean of V."""
    rng = np.random.default_rng(2)
    q = _f16(rng, (1, 2, 1, 32))
    k = _f16(rng, (1, 1, 50, 32))
    v = _f16(rng, (1, 1, 50, 32))
    np.testing.assert_array_equal(O.attention_kv(q, k, v, causal=True), O.attention_kv(q, k, v))
    z = np.zeros_like(q)
    np.testing.assert_allclose(O.attention_kv(z, k, v, causal=True)[0, 0, 0],
                               v[0, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-13)


def test_rejects_more_queries_than_keys():
    rng = np.random.default_rng(3)
    with pytest.raises(RuntimeError):
        O.attention_kv(_f16(rng, (1, 1, 5, 16)), _f16(rng, (1, 1, 4, 16)), _f16(rng, (1, 1, 4, 16)))


@pytest.mark.parametrize("causal", [False, True])
def test_quant_kv_square_case_equals_square_model(causal):
    rng = np.random.default_rng(4)
    S = 200
    q = _f16(rng, (1, 4, S, 64))
    k = _f16(rng, (1, 2, S, 64), offset=rng.standard_normal(64) * 3)
    v = _f16(rng, (1, 2, S, 64))
    qz = O.quantize_qk(q, k)
    qi, qs = O.quantize_q(q)
    assert np.array_equal(qi, qz["q_i8"]) and np.array_equal(qs, qz["q_scale"])
    kc = O.quantize_k_cache(k)
    assert np.array_equal(kc["k_i8"], qz["k_i8"]) and np.array_equal(kc["k_scale"], qz["k_scale"])
    a = O.quant_attention_kv(qi, qs, kc, v, causal=causal)
    b = O.quant_attention(qz, v, causal=causal)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("Sq", [1, 5, 32])
def test_quant_kv_decode_rows_are_last_rows_of_prefill_model(Sq):
    """With Sk - Sq a multiple of 128, the decode rows form exactly the last Q
    block of the prefill, so their quantisation and scores coincide."""
    rng = np.random.default_rng(10 + Sq)
    Sk = 256 + Sq
    q_full = _f16(rng, (1, 4, Sk, 64))
    k = _f16(rng, (1, 2, Sk, 64), offset=rng.standard_normal(64) * 3)
    v = _f16(rng, (1, 2, Sk, 64))
    qz = O.quantize_qk(q_full, k)
    qi, qs = O.quantize_q(q_full[:, :, Sk - Sq:])
    assert np.array_equal(qi, qz["q_i8"][:, :, Sk - Sq:])
    assert np.array_equal(qs[..., 0], qz["q_scale"][..., -1])
    dec = O.quant_attention_kv(qi, qs, O.quantize_k_cache(k), v, causal=True)
    ref = O.quant_attention(qz, v, causal=True, rows=np.arange(Sk - Sq, Sk))
    np.testing.assert_allclose(dec, ref, rtol=0, atol=1e-13)


def test_quant_kv_lossless_grid_equals_exact():
    """Q, K on exact INT8 grids with zero channel means: the quantised decode
    model equals exact decode attention up to the fp16 rounding of P."""
    rng = np.random.default_rng(20)
    Sq, Sk, D = 4, 512, 64
    q = np.zeros((1, 2, Sq, D))
    blk = rng.integers(-127, 128, (Sq, D)).astype(np.float64)
    blk[0, 0] = 127
    q[0, 0] = blk * 2.0 ** -4
    q[0, 1] = -blk * 2.0 ** -5
    k = np.zeros((1, 1, Sk, D))
    ints = rng.integers(-127, 128, (Sk // 2, D)).astype(np.float64)
    ints[::64, 0] = -127
    k[0, 0, :Sk // 2] = ints
    k[0, 0, Sk // 2:] = -ints
    for b0 in range(0, Sk, 64):
        k[0, 0, b0:b0 + 64] *= 2.0 ** -(3 + (b0 // 64) % 4)
    q, k = q.astype(np.float16), k.astype(np.float16)
    v = rng.standard_normal((1, 1, Sk, D)).astype(np.float16)
    kc = O.quantize_k_cache(k)
    assert not kc["k_mean"].any()
    qi, qs = O.quantize_q(q)
    o_q, l_q = O.quant_attention_kv(qi, qs, kc, v, causal=True, with_lse=True)
    o_e, l_e = O.attention_kv(q, k, v, causal=True, with_lse=True)
    np.testing.assert_allclose(l_q, l_e, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_q, o_e, rtol=0, atol=2e-3)
