"""Pins for the oracle's router gating GEMM, routing from it, and the
shared-expert gate of the combine.

* brute force: each logit as a math.fsum dot product over weights decoded
  independently (golden e2m1 table, torch's e4m3), on a tiny router with a
  gate row;
* closed forms: a power-of-two scale2 scales every logit exactly; all-zero
  codes give zero logits; the gate row changes only the gate logit;
* routing from the router is route_topk of its logits as fp32 values;
* the gated combine: a zero gate logit halves the shared expert's
  contribution, and the factor is scipy's logistic function.
"""
import math
import operator

import numpy as np
import scipy.special
import torch

import oracle
from _golden import lines
from oracle.ffn import bf16_bits_to_f64
from workloads import make_router, make_workload


def _e2m1_table():
    return {int(c): float(v) for c, v in (ln.split() for ln in lines("e2m1_codes.txt"))}


def _decode_rows(codes, scales, s2):
    e2 = _e2m1_table()
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    rows = []
    for n in range(codes.shape[0]):
        row = []
        for j in range(codes.shape[1]):
            b = int(codes[n, j])
            for k, c in ((2 * j, b & 0xF), (2 * j + 1, b >> 4)):
                row.append(e2[c] * float(sc[n, k // 16]) * float(s2))
        rows.append(row)
    return rows


def test_logits_match_fsum_brute_force():
    wl = make_workload("r", T=3, H=64, E=5, K=2, I=32, has_shared=True, seed=1,
                       with_weights=False)
    rb = make_router(5, 64, True, seed=1, scale2=0.375)
    got = oracle.router_logits(wl.x_bf16, rb.codes, rb.scales, rb.scale2)
    W = _decode_rows(rb.codes, rb.scales, rb.scale2)
    x = bf16_bits_to_f64(wl.x_bf16).tolist()
    assert got.shape == (3, 6)
    for t in range(3):
        for e in range(6):
            want = math.fsum(map(operator.mul, x[t], W[e]))
            assert abs(got[t, e] - want) <= 1e-12 * max(1.0, abs(want))


def test_scale2_power_of_two_and_zero_codes():
    wl = make_workload("r", T=7, H=256, E=8, K=2, I=32, has_shared=False, seed=2,
                       with_weights=False)
    rb = make_router(8, 256, False, seed=2)
    a = oracle.router_logits(wl.x_bf16, rb.codes, rb.scales, rb.scale2)
    b = oracle.router_logits(wl.x_bf16, rb.codes, rb.scales, rb.scale2 * 16.0)
    assert np.array_equal(b, 16.0 * a)
    z = oracle.router_logits(wl.x_bf16, np.zeros_like(rb.codes), rb.scales, rb.scale2)
    assert np.all(z == 0.0)


def test_gate_row_only_feeds_the_gate():
    wl = make_workload("r", T=9, H=256, E=16, K=4, I=32, has_shared=True, seed=3,
                       with_weights=False)
    rb = make_router(16, 256, True, seed=3)
    ids, w, z, gate = oracle.router_route(wl.x_bf16, rb.codes, rb.scales, rb.scale2, 16, 4)
    codes2 = rb.codes.copy()
    codes2[16] ^= 0x11
    ids2, w2, z2, gate2 = oracle.router_route(wl.x_bf16, codes2, rb.scales, rb.scale2, 16, 4)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2) and np.array_equal(z, z2)
    assert not np.array_equal(gate, gate2)
    ids_r, w_r = oracle.route_topk(z.astype(np.float32), 4)
    assert np.array_equal(ids, ids_r) and np.array_equal(w, w_r)


def test_router_logits_have_unit_scale_at_the_layer_size():
    wl = make_workload("r", T=256, H=2048, E=512, K=10, I=32, has_shared=True, seed=0,
                       with_weights=False)
    rb = make_router(512, 2048, True, seed=0)
    z = oracle.router_logits(wl.x_bf16, rb.codes, rb.scales, rb.scale2)
    assert 0.4 < np.std(z) < 2.5


def test_gated_combine():
    rng = np.random.default_rng(4)
    T, K, H = 5, 3, 8
    y = rng.normal(size=(T * K + T, H))
    w = rng.random((T, K))
    slot_pos = np.arange(T * K + T)
    plain = oracle.combine(y, w, slot_pos, T, K, True)
    routed = oracle.combine(y, w, slot_pos, T, K, False)
    half = oracle.combine(y, w, slot_pos, T, K, True, shared_gate=np.zeros(T))
    np.testing.assert_allclose(half, routed + 0.5 * (plain - routed), rtol=1e-14, atol=1e-14)
    g = np.array([-30.0, -1.0, 0.25, 2.0, 40.0])
    gated = oracle.combine(y, w, slot_pos, T, K, True, shared_gate=g)
    want = routed + scipy.special.expit(g)[:, None] * (plain - routed)
    np.testing.assert_allclose(gated, want, rtol=1e-13, atol=1e-14)
