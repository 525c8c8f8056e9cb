"""Pins for the MX re-encoding of the bounded-error study (oracle/mx.py):
brute-force e2m1 rounding against the golden e2m1 table, the two scale rules'
closed forms, exactness of NVFP4 blocks that are already MX values, and the
per-element error bound of the re-encoding."""
import numpy as np
import pytest

from _golden import lines
from oracle.formats import dequant_nvfp4
from oracle.mx import e2m1_encode_rne_sat, mx_quant, mx_scale, nvfp4_as_mxfp4
from oracle.mx_study import study
from workloads import make_weights, make_workload


def _grid():
    vals = {int(c): float(v) for c, v in (ln.split() for ln in lines("e2m1_codes.txt"))}
    return sorted((vals[c], c) for c in range(8))


def _brute(v):
    """Nearest of the table's non-negative values by exhaustive search, the
    even code on a tie, 6 for anything beyond."""
    a = min(abs(v), 6.0)
    best = None
    for val, code in _grid():
        d = abs(a - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[2] % 2 == 1):
            best = (d, val, code)
    return -best[1] if v < 0 else best[1]


def test_e2m1_rounding_brute_force_midpoints_and_saturation():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-8, 8, 3000),
                        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 100.0, 0.0],
                        -np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])])
    got = e2m1_encode_rne_sat(v)
    want = np.array([_brute(float(t)) for t in v])
    assert np.array_equal(got, want)
    # the ties by hand: the even code wins
    assert list(e2m1_encode_rne_sat([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])) == [0, 1, 1, 2, 2, 4, 4]


def test_scale_rules_closed_forms():
    # e2m1 (max 6 = 1.5 * 2**2): "ocp" X = 2**(floor(log2 amax) - 2); "fit" the
    # smallest power of two with amax / X <= 6
    assert list(mx_scale([6.0, 7.0, 0.75, 4.0, 0.0], "e2m1", "ocp")) == [1.0, 1.0, 0.125, 1.0, 1.0]
    assert list(mx_scale([6.0, 7.0, 0.75, 4.0, 0.0], "e2m1", "fit")) == [1.0, 2.0, 0.125, 1.0, 1.0]
    # e4m3 (max 448 = 1.75 * 2**8)
    assert list(mx_scale([448.0, 500.0, 1.0], "e4m3", "ocp")) == [1.0, 1.0, 2.0 ** -8]
    assert list(mx_scale([448.0, 500.0, 1.0], "e4m3", "fit")) == [1.0, 2.0, 2.0 ** -8]
    # a value above the element maximum saturates under "ocp" only
    b = np.full((1, 32), 0.5)
    b[0, 0] = 7.0
    assert mx_quant(b, "e2m1", "ocp")[0, 0] == 6.0
    assert mx_quant(b, "e2m1", "fit")[0, 0] == 8.0


@pytest.mark.parametrize("rule", ["ocp", "fit"])
def test_nvfp4_blocks_that_are_mx_values_survive(rule):
    """Both e4m3 scales of a 32-block equal to one power of two: the values
    are e2m1 x 2**k, which MXFP4 holds exactly under either rule."""
    rng = np.random.default_rng(3)
    N, K = 16, 256
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    # e4m3 codes with mantissa 0: 2**(e - 7); one exponent per 32-block
    e = rng.integers(3, 12, size=(N, K // 32))
    scales = np.repeat((e << 3).astype(np.uint8), 2, axis=1)
    w = dequant_nvfp4(codes, scales, 1.0)
    assert np.array_equal(nvfp4_as_mxfp4(codes, scales, rule), w)


@pytest.mark.parametrize("rule", ["ocp", "fit"])
def test_reencoding_error_bound(rule):
    """Each element lands within half an e2m1 grid step of its source (the
    step is 0.5, 1 or 2 X below 2X, 4X and 6X), or at the saturation value."""
    bank = make_weights(2, 256, 128, False, seed=5)
    w = dequant_nvfp4(bank.gu_codes[0], bank.gu_scales[0], 1.0)
    m = nvfp4_as_mxfp4(bank.gu_codes[0], bank.gu_scales[0], rule)
    b = w.reshape(w.shape[0], -1, 32)
    X = mx_scale(np.abs(b).max(axis=-1), "e2m1", rule)[..., None]
    a = np.abs(b) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = X * np.where(a > 6, a - 6, step / 2)
    assert np.all(np.abs(m.reshape(b.shape) - b) <= bound * (1 + 1e-12))


def test_study_runs_and_ranks_the_arms():
    """On a small layer: exact encodings give zero error, and the FP4
    weights cost more than the FP8 activations (they hold 2 significant bits
    of the 6 an NVFP4 weight can have)."""
    wl = make_workload("mx", T=6, H=256, E=8, K=2, I=128, has_shared=True, seed=6)
    res = study(wl)
    assert all(np.isfinite(v) for v in res.values())
    assert res["W_mxfp4[fit]"] > res["x_mxfp8[fit]"]
    assert res["full_mx[fit]"] >= res["xh_mxfp8[fit]"] * 0.5
