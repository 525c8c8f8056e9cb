"""Pins for the oracle's bf16 helpers, which the tight parity gate rests on.

* ``bf16_bits_to_f64`` (the activations as the oracle reads them) against the
  format's closed form evaluated with ``math.ldexp`` on all 65,536 patterns,
  and against hand-worked patterns (tests/golden/bf16_values.txt);
* ``_round_bf16`` (where the rounding oracle stores h and y in bf16) against
  hand-worked ties, subnormals and overflow (tests/golden/bf16_rounding.txt),
  and against a brute-force nearest-value search over every finite bf16 value
  with ties to the even pattern.
"""
import math

import numpy as np

from _golden import table
from oracle.ffn import _round_bf16, bf16_bits_to_f64

_ENV = {"inf": math.inf, "nan": math.nan}


def _closed_form(b: int) -> float:
    s, e, m = b >> 15, (b >> 7) & 0xFF, b & 0x7F
    if e == 0xFF:
        v = math.inf if m == 0 else math.nan
    elif e == 0:
        v = math.ldexp(m, -133)                 # m/128 * 2^-126
    else:
        v = math.ldexp(128 + m, e - 127 - 7)    # (1 + m/128) * 2^(e-127)
    return -v if s else v


def _same(a: float, b: float) -> bool:
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_bf16_decode_all_patterns_match_the_closed_form():
    got = bf16_bits_to_f64(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    for b in range(65536):
        assert _same(float(got[b]), _closed_form(b)), hex(b)


def test_bf16_decode_hand_worked_patterns():
    rows = table("bf16_values.txt")
    assert len(rows) >= 10
    bits = np.array([int(h, 16) for h, _ in rows], dtype=np.uint16)
    got = bf16_bits_to_f64(bits)
    for (h, v), g in zip(rows, got):
        assert _same(float(g), float(eval(v, {}, _ENV))), h


def test_round_bf16_hand_worked_values():
    rows = table("bf16_rounding.txt")
    src = np.array([float(eval(a, {}, _ENV)) for a, _ in rows])
    assert np.array_equal(src.astype(np.float32).astype(np.float64), src)   # exact in fp32
    got = _round_bf16(src)
    for (a, b), g in zip(rows, got):
        assert _same(float(g), float(eval(b, {}, _ENV))), a


def _finite_bf16_table():
    """Every finite bf16 value >= 0 in ascending order, with its pattern (the
    patterns 0x0000..0x7F7F ascend with the value)."""
    pats = np.arange(0x7F80, dtype=np.int64)
    vals = np.array([_closed_form(int(p)) for p in pats])
    assert np.all(np.diff(vals) > 0)
    return pats, vals


def test_round_bf16_matches_nearest_value_search():
    pats, vals = _finite_bf16_table()
    top = vals[-1]
    half_ulp_top = (vals[-1] - vals[-2]) / 2          # spacing of the top binade
    rng = np.random.default_rng(7)
    # float32 values over the whole exponent range, subnormals included, plus
    # exact midpoints between bf16 neighbours of random patterns
    f = rng.integers(0, 0x7F800000, 200000, dtype=np.uint32).view(np.float32).astype(np.float64)
    i = rng.integers(0, vals.size - 1, 20000)
    mids = (vals[i] + vals[i + 1]) / 2
    a = np.concatenate([f, mids, [top + half_ulp_top, top + half_ulp_top / 2]])
    a = a[a.astype(np.float32).astype(np.float64) == a]            # exact in fp32
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, vals.size - 1)
    lo = np.clip(hi - 1, 0, vals.size - 1)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_lo = (lo != hi) & ((d_lo < d_hi) | ((d_lo == d_hi) & (pats[lo] % 2 == 0)))
    want = np.where(pick_lo, vals[lo], vals[hi])
    want = np.where(a >= top + half_ulp_top, np.inf, np.where(a > top, top, want))
    sign = np.where(rng.random(a.size) < 0.5, -1.0, 1.0)
    got = _round_bf16(sign * a)
    assert np.array_equal(got, sign * want)
