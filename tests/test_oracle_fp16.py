"""Pins of the oracle's binary16 conversions against numpy's float16 (an independent
library routine implementing the same IEEE-754 rounding)."""
import numpy as np


def test_f16_to_f32_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_random_patterns(orc):
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    got = orc.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_f16_dense_in_range(orc):
    # every 61st fp32 pattern between 2^-26 and 2^17, both signs: covers subnormal,
    # normal, the carry into the next binade and overflow to infinity
    lo = np.float32(2.0 ** -26).view(np.uint32)
    hi = np.float32(2.0 ** 17).view(np.uint32)
    u = np.arange(lo, hi, 61, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([u.view(np.float32), -u.view(np.float32)])
    got = orc.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_f16_ties_and_edges(orc):
    vals = np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 2.0 ** -24, 2.0 ** -25,
                     3 * 2.0 ** -26, 2.0 ** -25 + 2.0 ** -40, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -30,
                     1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, -2049.0],
                    dtype=np.float32)
    got = orc.f32_to_f16_bits(vals)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    # ties go to the even neighbour
    assert got[11] == np.float16(1.0).view(np.uint16)
    assert orc.f16_bits_to_f32(got[[13, 14]]).tolist() == [2048.0, 2052.0]
