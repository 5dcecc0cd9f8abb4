"""Pins for the oracle's binary16 conversions against numpy's float16, a library
implementation of IEEE 754 binary16 with round-to-nearest-even."""
import numpy as np

import oracle


def test_f16_decode_all_codes_match_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64_array(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero keeps its sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _f16_values():
    pos = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    return pos.view(np.float16).astype(np.float64)


def test_f16_encode_ties_and_neighbours_match_numpy():
    v = _f16_values()
    mids = (v[:-1] + v[1:]) / 2  # exact midpoints: every one is an f32 value
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    for arr in (mids32[::7], up[::7], dn[::7], v.astype(np.float32)[::5]):
        arr = np.concatenate([arr, -arr])
        ref = arr.astype(np.float16).view(np.uint16)
        got = oracle.f32_to_f16_array(arr)
        assert np.array_equal(got, ref)


def test_f16_encode_boundaries_match_numpy():
    special = np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e9, np.inf, -np.inf,
                        2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26,
                        3 * 2.0 ** -26, 6.0e-5, 6.1e-5, 1.0, 1.0 / 127.0],
                       dtype=np.float32)
    special = np.concatenate([special, -special])
    ref = special.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16_array(special)
    assert np.array_equal(got, ref)
    assert oracle.f32_to_f16(float("nan")) & 0x7C00 == 0x7C00


def test_f16_encode_random_match_numpy():
    rng = np.random.default_rng(1)
    mant = rng.random(20000, dtype=np.float32) + np.float32(1.0)
    expo = rng.integers(-30, 18, size=20000)
    x = (mant * np.exp2(expo).astype(np.float32)).astype(np.float32)
    x = np.where(rng.random(20000) < 0.5, -x, x).astype(np.float32)
    ref = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16_array(x)
    assert np.array_equal(got, ref)
