"""Host check of the rounding identity the INT8 quantisers use to form codes
(no GPU): the fused-Q forward kernel on fp16 Q, and the standalone quantiser
on fp16 Q and on the smoothed K (fp32 values x = fp32(k) - mu).

The kernel quantises x (fp16) with r = fp32(127 / a), a = max|x| of the block,
as the low byte of fp32(fp32(x * r) + 1.5 * 2^23) instead of
clamp(rint(fp32(x * r)), -127, 127) (the SageAttention article's per-block
INT8 rule, as the standalone quantiser and the oracle compute it).  The
identity holds because |x * r| <= 127 (1 + 2^-23) < 127.5 when |x| <= a, so the
clamp never acts, and because in [2^23, 2^24) the fp32 spacing is 1: adding
1.5 * 2^23 rounds to an integer, to nearest with ties to even as rint does,
and the integer sits in the low mantissa bits.  Checked for every fp16 x with
|x| <= a, over many block maxima a (all finite fp16 magnitude patterns in a
stride, plus the extremes), and the fp16 maximum of the |x| bit patterns
against the float maximum.
"""
import numpy as np

MAGIC = np.float32(12582912.0)   # 1.5 * 2^23


def _codes_rule(x32, r):
    t = (x32 * r).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int64)


def _codes_kernel(x32, r):
    t = (x32 * r).astype(np.float32)
    u = (t + MAGIC).astype(np.float32).view(np.uint32)
    return (u & 0xFF).astype(np.uint8).view(np.int8).astype(np.int64)


def test_magic_rounding_matches_rint_and_clamp():
    bits = np.arange(0x7C00, dtype=np.uint16)            # every finite non-negative fp16 pattern
    mags = bits.view(np.float16)
    all_x = np.concatenate([mags, -mags]).astype(np.float32)
    amaxes = np.concatenate([bits[1::97], bits[-8:], bits[1:8]])
    for ab in amaxes:
        a = np.float32(np.uint16(ab).view(np.float16))
        r = np.float32(np.float32(127.0) / a)
        x = all_x[np.abs(all_x) <= a]
        assert np.array_equal(_codes_kernel(x, r), _codes_rule(x, r)), float(a)


def test_ties_round_to_even():
    r = np.float32(1.0)
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5], np.float32)
    assert list(_codes_kernel(x, r)) == [0, 2, 2, 0, -2, -2, 126, -126]


def test_bit_pattern_maximum_is_magnitude_maximum():
    rng = np.random.default_rng(0)
    for _ in range(200):
        h = rng.standard_normal(256).astype(np.float16) * np.float16(rng.uniform(0.01, 100))
        pat = (h.view(np.uint16) & 0x7FFF)
        assert np.uint16(pat.max()).view(np.float16) == np.abs(h).max()


def test_identity_for_fp32_values():
    """The standalone quantiser applies the same identity to the smoothed K,
    whose values are fp32 numbers (fp32(k) - mu); checked on random fp32 x with
    |x| <= a over a spread of block maxima, with the maximum itself, its
    negative, exact half-way products and zero in every set."""
    rng = np.random.default_rng(7)
    for a in np.float32(2.0) ** rng.uniform(-20, 17, 300).astype(np.float32):
        a = np.float32(a)
        r = np.float32(np.float32(127.0) / a)
        x = (rng.uniform(-1, 1, 4000) * a).astype(np.float32)
        # products landing on n + 1/2 exactly (ties), where representable
        halves = (np.arange(-127, 127) + np.float32(0.5)).astype(np.float32) / r
        x = np.concatenate([x, [a, -a, np.float32(0)], halves[np.abs(halves) <= a].astype(np.float32)])
        assert np.array_equal(_codes_kernel(x, r), _codes_rule(x, r)), a

