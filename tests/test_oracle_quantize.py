"""Pins for the oracle's q8 activation quantizer (O2) by properties the q8 block
definition fixes, not by re-deriving its arithmetic:
round-trip error within half a step, the largest element on the grid end, sign
symmetry, power-of-two scale invariance, ties to even, the zero block, and the
scaled sum agreeing with the stored scale times the sum of the codes."""
import numpy as np
import pytest

import oracle
import synth


def _vals(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


@pytest.fixture(scope="module")
def data():
    rng = np.random.default_rng(7)
    x = synth.activations(rng, 24, 1024, outliers=True)
    return x, oracle.quantize(x)


def test_scale_is_f16_of_amax_over_127(data):
    x, (q, dh, s) = data
    amax = np.abs(x.reshape(x.shape[0], -1, 32)).max(axis=2).astype(np.float32)
    ref = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(dh, ref)


def test_round_trip_within_half_step(data):
    x, (q, dh, s) = data
    d = np.repeat(_vals(dh), 32, axis=1)
    err = np.abs(x.astype(np.float64) - d * q.astype(np.float64))
    unclamped = np.abs(q) < 127
    # half a step, plus the rounding of the binary32 quotient (|quotient| < 128)
    assert np.all(err[unclamped] <= d[unclamped] * (0.5 + 128 * 2.0 ** -24))
    # clamped codes sit at the end of the grid and the error is bounded by the
    # scale's own f16 rounding: |x| <= amax = 127 * d32, |d32 - dh| <= dh * 2^-11
    clamped = ~unclamped
    assert np.all(err[clamped] <= 127 * d[clamped] * 2.0 ** -10 + d[clamped] * 0.5)


def test_largest_element_maps_to_grid_end(data):
    x, (q, dh, s) = data
    xb = x.reshape(x.shape[0], -1, 32)
    qb = q.reshape(q.shape[0], -1, 32)
    idx = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, idx[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.abs(q) <= 127)


def test_scaled_sum_is_f16_of_scale_times_code_sum(data):
    x, (q, dh, s) = data
    S = q.reshape(q.shape[0], -1, 32).astype(np.int64).sum(axis=2)
    exact = _vals(dh) * S
    sv = _vals(s)
    ulp = np.spacing(np.abs(sv).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(sv - exact) <= ulp / 2)


def test_sign_symmetry(data):
    x, (q, dh, s) = data
    qn, dhn, sn = oracle.quantize(-x)
    assert np.array_equal(qn, -q)
    assert np.array_equal(dhn, dh)
    assert np.array_equal(_vals(sn), -_vals(s))


@pytest.mark.parametrize("k", [-3, 2])
def test_power_of_two_scaling(data, k):
    x, (q, dh, s) = data
    xs = (x * np.float32(2.0 ** k)).astype(np.float32)
    qk, dhk, sk = oracle.quantize(xs)
    assert np.array_equal(qk, q)
    assert np.array_equal(_vals(dhk), _vals(dh) * 2.0 ** k)
    assert np.array_equal(_vals(sk), _vals(s) * 2.0 ** k)


def test_zero_and_vanishing_blocks():
    x = np.zeros((2, 64), np.float32)
    x[1, :32] = 1e-6  # amax / 127 rounds to 0 in binary16
    q, dh, s = oracle.quantize(x)
    assert not q.any() and not dh.any() and not s.any()


def test_ties_round_to_even():
    step = 0.0625  # amax = 127 * step gives dh = step exactly
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127 * step
    halves = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 126.5]
    x[0, 1:1 + len(halves)] = np.array(halves, np.float32) * np.float32(step)
    q, dh, s = oracle.quantize(x)
    assert _vals(dh)[0, 0] == step
    assert list(q[0, 1:1 + len(halves)]) == [0, 2, 2, 4, 0, -2, -2, 126]


def test_subnormal_scale():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2e-5          # amax / 127 is an f16 subnormal
    x[0, 1] = -1e-5
    q, dh, s = oracle.quantize(x)
    d = _vals(dh)[0, 0]
    assert 0 < d < 2.0 ** -14
    assert q[0, 0] == np.rint(np.float32(2e-5) / np.float32(d))
    assert abs(x[0, 1] - d * q[0, 1]) <= d / 2


def test_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.quantize(np.full((1, 32), np.nan, np.float32))
    with pytest.raises(ValueError):
        oracle.quantize(np.full((1, 32), 3000.0, np.float32))
