"""Properties of the seeded synthetic workloads (shapes, ranges, skew, outliers)."""
import numpy as np

import oracle
from workloads import CONFIGS, make_weights, workload_for
from workloads.generators import SCALE_CODE_HI, SCALE_CODE_LO, bf16_bits_to_f32


def test_tiny_is_deterministic_and_shaped():
    a = workload_for("tiny")
    b = workload_for("tiny")
    assert a.x_bf16.shape == (4, 256) and a.logits.shape == (4, 8)
    for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales", "scale2"):
        assert np.array_equal(getattr(a.weights, n), getattr(b.weights, n))
    W = a.weights
    assert W.gu_codes.shape == (8, 256, 128) and W.gu_scales.shape == (8, 256, 16)
    assert W.dn_codes.shape == (8, 256, 64) and W.dn_scales.shape == (8, 256, 8)
    assert np.all(W.scale2 == 1.0)
    assert W.bytes_per_expert == 55296


def test_scale_codes_span_2_to_the_minus_4_to_4():
    W = make_weights(16, 512, 128, True, seed=3)
    s = np.concatenate([W.gu_scales.ravel(), W.dn_scales.ravel()])
    assert s.min() == SCALE_CODE_LO and s.max() == SCALE_CODE_HI
    v = oracle.e4m3_decode(np.array([SCALE_CODE_LO, SCALE_CODE_HI]))
    assert v.tolist() == [2.0 ** -4, 4.0]
    nib = np.concatenate([W.gu_codes.ravel() & 15, W.gu_codes.ravel() >> 4])
    assert np.bincount(nib, minlength=16).min() > 0.9 * nib.size / 16


def test_full_size_expert_bytes():
    kw = CONFIGS["decode"]
    H, I = kw["H"], kw["I"]
    assert 2 * I * H // 2 + 2 * I * H // 16 + H * I // 2 + H * I // 16 == 1769472


def test_prefill_bias_and_x_distribution():
    w = workload_for("prefill", with_weights=False)
    assert w.x_bf16.shape == (4096, 2048)
    assert abs(np.std(w.meta["bias"]) - 0.5) < 0.05
    x = bf16_bits_to_f32(w.x_bf16)
    assert abs(x.std() - 1.0) < 0.01


def test_long_prefill_is_zipf_skewed():
    w = workload_for("long_prefill", with_weights=False)
    ids, _ = oracle.route_topk(w.logits, w.K)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    T = w.T
    assert (counts > 0.05 * T).sum() >= 5          # a few experts take > 5 % of the tokens
    assert (counts < 10).sum() >= 100              # many take fewer than 10
    assert counts.max() > 0.5 * T


def test_fp8_arm_heavy_tails_and_outliers():
    w = workload_for("fp8_arm", with_weights=False)
    x = bf16_bits_to_f32(w.x_bf16)
    n_out = int(round(1e-3 * w.T * w.H))
    assert (np.abs(x) > 100).sum() >= 0.5 * n_out
    assert np.abs(x).max() > 1000
