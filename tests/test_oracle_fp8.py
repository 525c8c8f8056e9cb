"""Pins for the per-token-row e4m3 quantiser of the FP8 activation arm."""
from fractions import Fraction

import numpy as np

import oracle
from _golden import table


def test_hand_worked_rows():
    for vals, s, codes in table("fp8_rows.txt"):
        x = np.array([[float(v) for v in vals.split()]], dtype=np.float32)
        q, sc = oracle.rowquant_e4m3(x)
        assert sc[0] == np.float32(float(s))
        assert q[0].tolist() == [int(c, 16) for c in codes.split()]


def _f32_nearest(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of a rational, by checking the neighbours of a float64 guess."""
    g = np.float32(float(fr))
    best = g
    for c in (np.nextafter(g, np.float32(-np.inf)), g, np.nextafter(g, np.float32(np.inf))):
        if abs(Fraction(float(c)) - fr) < abs(Fraction(float(best)) - fr):
            best = c
    return best


def test_scales_are_correctly_rounded_quotients():
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, (64, 48)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    q, s = oracle.rowquant_e4m3(x)
    for t in range(x.shape[0]):
        amax = Fraction(float(np.max(np.abs(x[t]))))
        assert s[t] == _f32_nearest(amax / 448)
        inv = _f32_nearest(448 / amax)
        v = np.array([_f32_nearest(Fraction(float(xi)) * Fraction(float(inv))) for xi in x[t]],
                     dtype=np.float32)
        assert np.array_equal(q[t], oracle.e4m3_encode_rne_sat(v))
    # the largest magnitude of each row lands on (or next to) the top code 448
    deq = oracle.e4m3_decode(q)
    assert np.all(np.max(np.abs(deq), axis=1) >= 416.0)


def test_dequantised_rows_are_within_the_e4m3_bound():
    rng = np.random.default_rng(6)
    x = rng.standard_t(3, (32, 256)).astype(np.float32)
    xd = oracle.rowquant_dequant(x)
    amax = np.max(np.abs(x), axis=1, keepdims=True)
    err = np.abs(xd - x)
    # normal range: half-ulp relative 2**-4; below 2**-6 of the row scale: absolute half-ulp 2**-10
    bound = np.maximum(np.abs(x) * 2.0 ** -4, amax / 448.0 * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
