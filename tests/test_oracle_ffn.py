"""Pins for the oracle's expert FFN, shared expert and combine.

* brute force: pure-Python math.fsum loops over independently decoded weights
  (golden e2m1 table, torch's e4m3) on the tiny layer and a tiny shared-expert
  layer;
* invariants that fix the structure: K=1 is the dense FFN of the chosen expert,
  token permutation permutes the output, expert relabelling leaves it unchanged,
  K=E is the softmax-weighted dense mixture, scale2 scales exactly, zero codes
  give zero, the shared expert adds the dense FFN of group E.
"""
import math
import operator

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.ffn import bf16_bits_to_f64
from _golden import lines
from workloads import make_workload, make_weights


def _e2m1_table():
    return {int(c): float(v) for c, v in (ln.split() for ln in lines("e2m1_codes.txt"))}


def _decode_matrix(codes, scales, s2):
    e2 = _e2m1_table()
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    N, Kh = codes.shape
    W = []
    for n in range(N):
        row = []
        for j in range(Kh):
            b = int(codes[n, j])
            for k, c in ((2 * j, b & 0xF), (2 * j + 1, b >> 4)):
                row.append(e2[c] * float(sc[n, k // 16]) * float(s2))
        W.append(row)
    return W


def _dot(a, b):
    return math.fsum(map(operator.mul, a, b))


def _brute_layer(w):
    T, H, E, K, I = w.T, w.H, w.E, w.K, w.I
    bank = w.weights
    x = bf16_bits_to_f64(w.x_bf16).tolist()
    out = [[0.0] * H for _ in range(T)]
    terms = [[[] for _ in range(H)] for _ in range(T)]
    dense = {}

    def ffn(e, xr):
        if e not in dense:
            s2 = bank.scale2[e]
            dense[e] = (_decode_matrix(bank.gu_codes[e], bank.gu_scales[e], 1.0),
                        _decode_matrix(bank.dn_codes[e], bank.dn_scales[e], s2[2]), s2)
        gu, dn, s2 = dense[e]
        g = [_dot(xr, gu[j]) * float(s2[0]) for j in range(I)]
        u = [_dot(xr, gu[I + j]) * float(s2[1]) for j in range(I)]
        h = [gi * float(scipy.special.expit(gi)) * ui for gi, ui in zip(g, u)]
        return [_dot(h, dn[n]) for n in range(H)]

    for t in range(T):
        z = [(-math.inf if math.isnan(v) else float(v)) for v in w.logits[t]]
        order = sorted(range(E), key=lambda i: (-z[i], i))[:K]
        zs = [z[i] for i in order]
        ex = [math.exp(v - zs[0]) for v in zs]
        tot = math.fsum(ex)
        for e, wt in zip(order, (v / tot for v in ex)):
            y = ffn(e, x[t])
            for n in range(H):
                terms[t][n].append(wt * y[n])
        if w.has_shared:
            y = ffn(E, x[t])
            for n in range(H):
                terms[t][n].append(y[n])
        for n in range(H):
            out[t][n] = math.fsum(terms[t][n])
    return np.array(out)


@pytest.mark.parametrize("cfg", [
    dict(T=4, H=256, E=8, K=2, I=128, has_shared=False),           # the tiny layer
    dict(T=5, H=64, E=6, K=3, I=32, has_shared=True),
])
def test_layer_matches_fsum_brute_force(cfg):
    w = make_workload("t", seed=0, **cfg)
    if cfg["has_shared"]:
        w.weights.scale2[:] = np.array([0.5, 2.0, 0.25], dtype=np.float32)
    ref = _brute_layer(w)
    got = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K)["out"]
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def _wl(T=6, H=64, E=8, K=2, I=32, has_shared=False, seed=1):
    return make_workload("inv", T=T, H=H, E=E, K=K, I=I, has_shared=has_shared, seed=seed)


def _rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


def test_top1_equals_dense_ffn_of_chosen_expert():
    w = _wl(K=1)
    r = oracle.moe_layer(w.x_bf16, w.logits, w.weights, 1)
    assert np.all(r["w"] == 1.0)
    x = bf16_bits_to_f64(w.x_bf16)
    for t in range(w.T):
        e = int(r["ids"][t, 0])
        wg, wu, wd = oracle.ffn.dequant_expert(w.weights, e)
        dense = oracle.silu(x[t] @ wg.T) * (x[t] @ wu.T) @ wd.T
        assert _rel(r["out"][t], dense) <= 1e-13


def test_token_permutation_permutes_outputs():
    w = _wl(T=9, has_shared=True)
    p = np.random.default_rng(0).permutation(w.T)
    a = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K)["out"]
    b = oracle.moe_layer(w.x_bf16[p], w.logits[p], w.weights, w.K)["out"]
    assert _rel(b, a[p]) <= 1e-13


def test_expert_relabelling_leaves_output_unchanged():
    w = _wl(T=7, E=8, K=3, has_shared=True)
    bank = w.weights
    pi = np.random.default_rng(1).permutation(w.E)
    full = np.concatenate([pi, [w.E]])                 # the shared expert keeps index E
    relab = make_weights(w.E, w.H, w.I, True, seed=1)
    for name in ("gu_codes", "gu_scales", "dn_codes", "dn_scales", "scale2"):
        setattr(relab, name, getattr(bank, name)[full])
    a = oracle.moe_layer(w.x_bf16, w.logits, bank, w.K)["out"]
    b = oracle.moe_layer(w.x_bf16, w.logits[:, pi], relab, w.K)["out"]
    assert _rel(b, a) <= 1e-13


def test_k_equal_e_is_the_softmax_weighted_dense_mixture():
    w = _wl(T=5, E=8, K=8)
    r = oracle.moe_layer(w.x_bf16, w.logits, w.weights, 8)
    x = bf16_bits_to_f64(w.x_bf16)
    p = scipy.special.softmax(w.logits.astype(np.float64), axis=1)
    mix = np.zeros_like(r["out"])
    for e in range(w.E):
        wg, wu, wd = oracle.ffn.dequant_expert(w.weights, e)
        mix += p[:, e:e + 1] * (oracle.silu(x @ wg.T) * (x @ wu.T) @ wd.T)
    assert _rel(r["out"], mix) <= 1e-12


def test_scale2_down_power_of_two_scales_output_exactly():
    w = _wl(has_shared=True)
    a = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K)["out"]
    w.weights.scale2[:, 2] *= np.float32(8.0)
    b = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K)["out"]
    assert np.array_equal(b, 8.0 * a)


def test_scale2_gate_and_up_enter_as_weight_factors():
    w = _wl()
    x = bf16_bits_to_f64(w.x_bf16)
    w.weights.scale2[3] = np.array([0.75, 3.0, 1.5], dtype=np.float32)
    wg, wu, wd = oracle.ffn.dequant_expert(w.weights, 3)
    w.weights.scale2[3] = 1.0
    g1, u1, d1 = oracle.ffn.dequant_expert(w.weights, 3)
    assert np.array_equal(wg, 0.75 * g1) and np.array_equal(wu, 3.0 * u1)
    assert np.array_equal(wd, 1.5 * d1)


def test_zero_codes_give_zero_output():
    w = _wl(has_shared=True)
    for name in ("gu_codes", "dn_codes"):
        getattr(w.weights, name)[:] = 0
    out = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K)["out"]
    assert np.all(out == 0.0)


def test_shared_expert_adds_dense_ffn_of_group_E():
    w = _wl(has_shared=True)
    with_shared = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K)["out"]
    w2 = _wl(has_shared=False)
    without = oracle.moe_layer(w2.x_bf16, w2.logits, w2.weights, w2.K)["out"]
    x = bf16_bits_to_f64(w.x_bf16)
    wg, wu, wd = oracle.ffn.dequant_expert(w.weights, w.E)
    dense = oracle.silu(x @ wg.T) * (x @ wu.T) @ wd.T
    # same seed, same routed experts: the shared bank only adds group E
    assert _rel(with_shared - without, dense) <= 1e-12


def test_silu_matches_scipy_expit_form():
    g = np.concatenate([np.linspace(-800, 800, 4001), [0.0, -0.0, 1e-300]])
    np.testing.assert_allclose(oracle.silu(g), g * scipy.special.expit(g), rtol=1e-15, atol=1e-300)


def test_fp8_arm_emulation_within_the_gate_on_heavy_tails():
    w = make_workload("f", T=16, H=256, E=8, K=2, I=64, has_shared=True, seed=2, x_kind="student_t")
    exact = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K)["out"]
    fp8 = oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K, act_mode="fp8_row")["out"]
    err = np.max(np.abs(fp8 - exact)) / np.max(np.abs(exact))
    assert 0 < err < 6e-2


def test_activation_arms_per_expert_class():
    """The per-class arms (the shared-expert A/B table's arm S and its
    mirror): routed slots carry exactly the outputs of the arm their class
    uses, shared slots those of the other, and without a shared expert
    "fp8_routed" is "fp8_row" and "fp8_shared" is "bf16"."""
    w = make_workload("arms", T=6, H=256, E=8, K=2, I=128, has_shared=True, seed=4)
    lay = {m: oracle.moe_layer(w.x_bf16, w.logits, w.weights, w.K, act_mode=m)
           for m in ("bf16", "fp8_row", "fp8_routed", "fp8_shared")}
    TK = w.T * w.K
    pos = lay["bf16"]["slot_pos"]
    routed, shared = pos[:TK], pos[TK:]
    for m, r_src, s_src in (("fp8_routed", "fp8_row", "bf16"), ("fp8_shared", "bf16", "fp8_row")):
        y = lay[m]["y_slots"]
        assert np.array_equal(y[routed], lay[r_src]["y_slots"][routed])
        assert np.array_equal(y[shared], lay[s_src]["y_slots"][shared])
        # the combine is linear in the shared rows
        want = lay[r_src]["out"] - lay[r_src]["y_slots"][shared] + lay[s_src]["y_slots"][shared]
        assert np.allclose(lay[m]["out"], want, rtol=0, atol=1e-12 * np.abs(want).max())
    assert not np.array_equal(lay["fp8_routed"]["out"], lay["fp8_row"]["out"])
    w0 = make_workload("arms0", T=6, H=256, E=8, K=2, I=128, has_shared=False, seed=4)
    o = {m: oracle.moe_layer(w0.x_bf16, w0.logits, w0.weights, w0.K, act_mode=m)["out"]
         for m in ("bf16", "fp8_row", "fp8_routed", "fp8_shared")}
    assert np.array_equal(o["fp8_routed"], o["fp8_row"])
    assert np.array_equal(o["fp8_shared"], o["bf16"])
