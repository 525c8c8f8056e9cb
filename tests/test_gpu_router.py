"""GPU parity of the fused router (router GEMM from an NVFP4 matrix + top-K)
and of the sigmoid-gated combine, against the fp64 oracle.

Gates:
  * logits and the gate logit: |z_gpu - z_exact| <= H * 2^-24 * sum_k |x_k W_ek|
    (recursive f32 summation of exact products, any order; the products
    themselves are exact: e2m1 x e4m3 x bf16 has <= 14 significant bits), plus
    the exact power-of-two scale2;
  * ids bit-exact against the oracle's top-K of the GPU's own logits (the
    router decides the integer ids in fp32, the precision of the logits);
  * weights within 4e-6 relative of the oracle's softmax of those logits;
  * the gated combine within one bf16 rounding of the fp64 sum on the GPU's
    own per-slot outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu import bf16_np, flush, setup, x_dev
from oracle.ffn import bf16_bits_to_f64
from oracle.formats import dequant_nvfp4
from workloads import DECODE_TS, make_router, make_workload, workload_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    return setup()


def _check_router(moe, x_bits, rb, K, tag):
    flush(f"router {tag}: T={x_bits.shape[0]} H={rb.H} E={rb.E} K={K} gate={rb.has_gate}")
    R = moe.NVFP4Router.from_bank(rb)
    x = x_dev(x_bits)
    ids, w, z, g = moe.moe_router_topk(R, x, K)
    ids2, w2, z2, g2 = moe.moe_router_topk(R, x, K)   # a second call: bitwise the same
    torch.cuda.synchronize()
    ids, w, z = ids.cpu().numpy(), w.cpu().numpy(), z.cpu().numpy()
    assert np.array_equal(ids, ids2.cpu().numpy()) and np.array_equal(w, w2.cpu().numpy())
    assert np.array_equal(z, z2.cpu().numpy())

    z_ref = oracle.router_logits(x_bits, rb.codes, rb.scales, rb.scale2)
    absw = np.abs(dequant_nvfp4(rb.codes, rb.scales, rb.scale2))
    bound = rb.H * 2.0 ** -24 * (np.abs(bf16_bits_to_f64(x_bits)) @ absw.T) + 1e-30
    err = np.abs(z.astype(np.float64) - z_ref[:, :rb.E])
    assert np.all(err <= bound[:, :rb.E]), f"max err/bound {np.max(err / bound[:, :rb.E]):.3g}"
    if rb.has_gate:
        g = g.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - z_ref[:, rb.E]) <= bound[:, rb.E])
        assert np.array_equal(g, g2.cpu().numpy().astype(np.float64))
    else:
        assert g is None

    ids_o, w_o = oracle.route_topk(z, K)
    assert np.array_equal(ids, ids_o)
    assert np.all(np.abs(w.astype(np.float64) - w_o) <= 4e-6 * w_o + 1e-30)
    # and the exact oracle routing agrees wherever the fp32 logits leave no
    # near-tie at the K-th place
    ids_x, _, _, _ = oracle.router_route(x_bits, rb.codes, rb.scales, rb.scale2, rb.E, K)
    zs = np.sort(z_ref[:, :rb.E], axis=1)[:, ::-1]
    gap = (zs[:, K - 1] - zs[:, K]) if rb.E > K else np.full(zs.shape[0], np.inf)
    clear = gap > 4 * np.max(bound[:, :rb.E], axis=1)
    assert np.array_equal(np.sort(ids[clear], axis=1), np.sort(ids_x[clear], axis=1))
    return ids, w, z, g


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "long_prefill", "fp8_arm"])
def test_router_on_configs(moe, name):
    Ts = DECODE_TS if name == "decode" else (None,)
    for T in Ts:
        wl = workload_for(name, T=T, with_weights=False)
        rb = make_router(wl.E, wl.H, wl.has_shared, seed=3)
        _check_router(moe, wl.x_bf16, rb, wl.K, f"{name}")


@pytest.mark.parametrize("E,H,T,K,gate", [
    (8, 256, 1, 1, False),       # smallest shapes: one k step, one 64-expert tile
    (100, 512, 37, 6, True),     # ragged E inside a 128 tile, ragged token tile
    (200, 256, 17, 8, False),    # 256-expert tile, padding rows
    (513, 2048, 33, 10, True),   # one past the 512 tile (the 1024-expert kernel)
    (1024, 256, 5, 32, True),    # maximum E and K
    (64, 8192, 3, 4, False),     # maximum H
    (1000, 512, 1024, 12, True), # largest T of the split-K kernel
    (100, 512, 1100, 6, True),   # 32-token tiled kernel: ragged T, E a multiple of 4
    (513, 256, 8200, 10, True),  # 64-token tiled kernel: E % 4 = 1, three expert tiles
    (1024, 256, 2000, 32, True), # tiled kernel at the maximum E and K
    (8, 8192, 1030, 2, False),   # tiled kernel at the maximum H and the smallest E
])
def test_router_edges(moe, E, H, T, K, gate):
    wl = make_workload("r", T=T, H=H, E=E, K=K, I=128, has_shared=gate, seed=5,
                       with_weights=False)
    rb = make_router(E, H, gate, seed=6)
    _check_router(moe, wl.x_bf16, rb, K, f"edge E={E}")


def test_router_zero_rows_and_ties(moe):
    """Zero activations give all-zero logits: every token picks experts
    0..K-1 (lower index first on ties) with equal weights 1/K."""
    T, H, E, K = 20, 512, 64, 8
    rb = make_router(E, H, True, seed=7)
    x = np.zeros((T, H), dtype=np.uint16)
    ids, w, z, g = _check_router(moe, x, rb, K, "zero rows")
    assert np.all(z == 0) and np.all(g == 0)
    assert np.array_equal(ids, np.tile(np.arange(K, dtype=np.int32), (T, 1)))
    assert np.all(w == np.float32(1.0 / K))


def test_gated_combine(moe):
    wl = make_workload("gated", T=37, H=256, E=8, K=2, I=128, has_shared=True, seed=9)
    rb = make_router(wl.E, wl.H, True, seed=8)
    W = moe.NVFP4Weights.from_bank(wl.weights)
    R = moe.NVFP4Router.from_bank(rb)
    x = x_dev(wl.x_bf16)
    ids, w, _, g = moe.moe_router_topk(R, x, wl.K)
    counts, offsets, sorted_slot, slot_pos, groups = moe.moe_permute(ids, wl.E, True)
    y = moe.moe_expert_ffn(W, x, wl.K, offsets, sorted_slot, groups)
    out = moe.moe_combine_gated(y, w, slot_pos, g, wl.K)
    plain = moe.moe_combine(y, w, slot_pos, wl.K, True)
    torch.cuda.synchronize()
    yn = bf16_np(y)
    gn = g.cpu().numpy().astype(np.float64)
    ref = oracle.combine(yn, w.cpu().numpy().astype(np.float64), slot_pos.cpu().numpy(), wl.T,
                         wl.K, True, shared_gate=gn)
    o = bf16_np(out)
    mag = np.max(np.abs(ref), axis=1, keepdims=True)
    assert np.all(np.abs(o - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * mag)
    # the gate changes the result (the sigmoid is not 1)
    assert not np.array_equal(o, bf16_np(plain))
    # a zero gate logit halves the shared expert exactly (sigmoid(0) = 1/2)
    zero = torch.zeros_like(g)
    half = moe.moe_combine_gated(y, w, slot_pos, zero, wl.K)
    torch.cuda.synchronize()
    ref_h = oracle.combine(yn, w.cpu().numpy().astype(np.float64), slot_pos.cpu().numpy(), wl.T,
                           wl.K, True, shared_gate=np.zeros(wl.T))
    assert np.all(np.abs(bf16_np(half) - ref_h) <= 2.0 ** -8 * np.abs(ref_h) + 1e-6 * mag)
