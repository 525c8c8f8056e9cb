"""GPU checks of the combined layer entry points: moe_route_permute (router
top-K and permutation in one kernel for batches of up to 8 tokens, the two
kernels above) and moe_expert_ffn_combine (FFN then combine in one call).
Both must reproduce the separate calls bit for bit -- they run the same
arithmetic in the same order -- and the layer through them must pass the same
oracle gates as the unfused one."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import bf16_np, flush, normwise, setup, x_dev
from workloads import DECODE_TS, make_workload, workload_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    return setup()


def _route_permute_both(moe, logits_np, K, E, has_shared):
    lg = torch.from_numpy(logits_np).cuda()
    fused = moe.moe_route_permute(lg, K, has_shared)
    ids, w = moe.moe_route_topk(lg, K)
    perm = moe.moe_permute(ids, E, has_shared)
    torch.cuda.synchronize()
    return fused, (ids, w) + tuple(perm)


@pytest.mark.parametrize("E", [8, 100, 200, 512, 1000])
@pytest.mark.parametrize("T", [1, 3, 4, 5, 8, 9, 16, 40])
def test_route_permute_matches_the_two_calls(moe, E, T):
    K = min(10, E)
    for hs in (False, True):
        wl = make_workload("rp", T=T, H=256, E=E, K=K, I=128, has_shared=hs, seed=T + E,
                           with_weights=False)
        fused, ref = _route_permute_both(moe, wl.logits, K, E, hs)
        names = ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "groups")
        for a, b, nm in zip(fused, ref, names):
            assert torch.equal(a, b), f"{nm} E={E} T={T} shared={hs}"
        # and the oracle's routing and permutation
        ids_o, _ = oracle.route_topk(wl.logits, K)
        assert np.array_equal(fused[0].cpu().numpy(), ids_o)
        want = oracle.permute(ids_o, E, hs)
        for g, w_, nm in zip(fused[2:6], want, names[2:6]):
            assert np.array_equal(g.cpu().numpy(), w_), nm


@pytest.mark.parametrize("E,K", [(1024, 32), (32, 32), (40, 32), (1, 1), (2, 2)])
def test_route_permute_largest_fused_batch(moe, E, K):
    """8 tokens x K = 32 (256 slots, one per thread of the fused block), with
    few experts (every group full) and the largest E."""
    for T in (7, 8):
        for hs in (False, True):
            wl = make_workload("rpk", T=T, H=256, E=E, K=K, I=128, has_shared=hs, seed=E + K,
                               with_weights=False)
            fused, ref = _route_permute_both(moe, wl.logits, K, E, hs)
            for a, b in zip(fused, ref):
                assert torch.equal(a, b), f"E={E} K={K} T={T} shared={hs}"
            ids_o, _ = oracle.route_topk(wl.logits, K)
            want = oracle.permute(ids_o, E, hs)
            for g, w_ in zip(fused[2:6], want):
                assert np.array_equal(g.cpu().numpy(), w_)


def test_route_permute_ties_and_nan(moe):
    T, E, K = 4, 64, 6
    lg = np.zeros((T, E), dtype=np.float32)
    lg[0, 10:20] = 1.0
    lg[1, 5] = np.nan
    lg[2, :] = -np.inf
    lg[3, ::2] = np.inf
    fused, ref = _route_permute_both(moe, lg, K, E, True)
    for a, b in zip(fused, ref):
        assert torch.equal(a, b)
    ids_o, _ = oracle.route_topk(lg, K)
    assert np.array_equal(fused[0].cpu().numpy(), ids_o)


def _ffn_combine_both(moe, wl, act_mode=0, gate=None, repeats=2):
    W = moe.NVFP4Weights.from_bank(wl.weights)
    x = x_dev(wl.x_bf16)
    ids, w, counts, offsets, sorted_slot, slot_pos, groups = moe.moe_route_permute(
        torch.from_numpy(wl.logits).cuda(), wl.K, wl.has_shared)
    y_ref = moe.moe_expert_ffn(W, x, wl.K, offsets, sorted_slot, groups, act_mode)
    out_ref = (moe.moe_combine(y_ref, w, slot_pos, wl.K, wl.has_shared) if gate is None
               else moe.moe_combine_gated(y_ref, w, slot_pos, gate, wl.K))
    ws = None
    outs = []
    for _ in range(repeats):  # repeated calls give the same bits
        y, out = moe.moe_expert_ffn_combine(W, x, wl.K, offsets, sorted_slot, groups, w, slot_pos,
                                            act_mode, gate=gate, ws=ws)
        outs.append((y.clone(), out.clone()))
    torch.cuda.synchronize()
    for y, out in outs:
        assert torch.equal(y, y_ref)
        assert torch.equal(out, out_ref)
    return outs[0][1], w, slot_pos


@pytest.mark.parametrize("T", DECODE_TS)
def test_ffn_combine_decode_full_size(moe, T):
    wl = workload_for("decode", T=T)
    flush(f"ffn_combine decode T={T}")
    out, w, slot_pos = _ffn_combine_both(moe, wl)
    # the fused layer against the exact oracle, with the unfused layer's gate
    exact = oracle.moe_layer(wl.x_bf16, wl.logits, wl.weights, wl.K)
    assert normwise(bf16_np(out), exact["out"]) <= 2e-2


@pytest.mark.parametrize("cfg", [
    dict(T=5, H=2048, E=64, K=10, I=512, has_shared=True),
    dict(T=8, H=256, E=4, K=2, I=128, has_shared=True),      # smallest H and I
    dict(T=7, H=4096, E=16, K=4, I=1024, has_shared=False),  # largest H and I
    dict(T=3, H=512, E=16, K=4, I=256, has_shared=False),
    dict(T=300, H=512, E=16, K=4, I=256, has_shared=True),   # the unfused (prefill) branch
])
def test_ffn_combine_shapes(moe, cfg):
    wl = make_workload("fc", seed=11, **cfg)
    flush(f"ffn_combine {cfg}")
    _ffn_combine_both(moe, wl)


def test_ffn_combine_fp8_and_gate(moe):
    wl = workload_for("decode", T=8)
    g = torch.from_numpy(np.linspace(-3, 3, wl.T).astype(np.float32)).cuda()
    _ffn_combine_both(moe, wl, act_mode=1)
    _ffn_combine_both(moe, wl, gate=g)
    _ffn_combine_both(moe, wl, act_mode=1, gate=g)


def test_ffn_combine_no_active_group(moe):
    """Every id out of range and no shared expert: no group is active, and
    the combine still writes the (all-zero) output."""
    wl = make_workload("na", T=4, H=512, E=16, K=4, I=256, has_shared=False, seed=3)
    W = moe.NVFP4Weights.from_bank(wl.weights)
    x = x_dev(wl.x_bf16)
    ids = torch.full((wl.T, wl.K), -1, dtype=torch.int32, device="cuda")
    w = torch.full((wl.T, wl.K), 0.25, dtype=torch.float32, device="cuda")
    counts, offsets, sorted_slot, slot_pos, groups = moe.moe_permute(ids, wl.E, False)
    out0 = torch.full((wl.T, wl.H), 7.0, dtype=torch.bfloat16, device="cuda")
    _, out = moe.moe_expert_ffn_combine(W, x, wl.K, offsets, sorted_slot, groups, w, slot_pos,
                                        out=out0)
    torch.cuda.synchronize()
    assert int(groups[0].item()) == 0
    assert torch.count_nonzero(out).item() == 0


def _gate_up_splits_k(wl):
    """Whether moe_expert_ffn splits the decode gate_up K over 4 waves for this
    launch (fewer than 2 gate_up units per CU, H / 128 a multiple of 4)."""
    if wl.T > 8:
        return False
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gmax = min(wl.T * wl.K + int(wl.has_shared), wl.E + int(wl.has_shared))
    return gmax * (wl.I // 16) < 2 * cus and (wl.H // 128) % 4 == 0


def _layer_split_k(wl, act_mode):
    """The K split of moe_layer's gate_up (1 = none), or None when the call
    takes the separate launches' path: when the largest possible block share
    of gate_up units is at most 4, the largest of 8, 4, 2 dividing H / 128
    whose waves (16 per CU) cover the share in one round."""
    nch, ncd = wl.H // 128, wl.I // 128
    if not (1 <= wl.T <= 8 and wl.E <= 1024 and wl.K <= 32 and act_mode in (0, 1)
            and wl.H % 128 == 0 and wl.I % 128 == 0 and nch in (2, 4, 8, 16) and ncd in (1, 2, 4, 8)):
        return None
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gmax = min(wl.T * wl.K + int(wl.has_shared), wl.E + int(wl.has_shared))
    share = -(-gmax * (wl.I // 16) // cus)
    ks = 1
    while share <= 4 and 2 * ks <= 8 and 2 * ks * share <= 16 and nch % (2 * ks) == 0:
        ks *= 2
    return ks


def _same_sums(wl, act_mode):
    """Whether the one-call layer and the separate launches add the gate_up
    products in the same order (the same K split, or the same path), so their
    outputs agree bit for bit."""
    ks = _layer_split_k(wl, act_mode)
    return ks is None or ks == (4 if _gate_up_splits_k(wl) else 1)


def _layer_vs_calls(moe, wl, act_mode=0, gate=None):
    W = moe.NVFP4Weights.from_bank(wl.weights)
    x = x_dev(wl.x_bf16)
    lg = torch.from_numpy(wl.logits).cuda()
    one = moe.moe_layer(W, x, lg, wl.K, act_mode, fused=True, gate=gate)
    again = moe.moe_layer(W, x, lg, wl.K, act_mode, fused=True, gate=gate)
    perm = moe.moe_route_permute(lg, wl.K, wl.has_shared)
    ids, w, counts, offsets, sorted_slot, slot_pos, groups = perm
    y_ref, out_ref = moe.moe_expert_ffn_combine(W, x, wl.K, offsets, sorted_slot, groups, w, slot_pos,
                                                act_mode, gate=gate)
    torch.cuda.synchronize()
    names = ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "groups")
    for nm, ref in zip(names, perm):
        assert torch.equal(one[nm], ref), nm
        assert torch.equal(again[nm], ref), nm
    assert torch.equal(one["y_slots"].view(torch.int16), again["y_slots"].view(torch.int16))
    assert torch.equal(one["out"].view(torch.int16), again["out"].view(torch.int16))
    # the layer's combine (inside the down launch for small batches) is the
    # combine kernel's arithmetic on the layer's own y rows, bit for bit
    out_c = (moe.moe_combine(one["y_slots"], one["w"], one["slot_pos"], wl.K, wl.has_shared)
             if gate is None else
             moe.moe_combine_gated(one["y_slots"], one["w"], one["slot_pos"], gate, wl.K))
    torch.cuda.synchronize()
    assert torch.equal(one["out"].view(torch.int16), out_c.view(torch.int16))
    if _same_sums(wl, act_mode):
        assert torch.equal(one["y_slots"].view(torch.int16), y_ref.view(torch.int16))
        assert torch.equal(one["out"].view(torch.int16), out_ref.view(torch.int16))
    else:  # another summation order: within a few bf16 roundings of each other
        assert normwise(bf16_np(one["out"]), bf16_np(out_ref)) <= 8e-3
    return one


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_layer_one_call_matches_the_calls(moe, T):
    """moe_layer (routing and permutation inside the gate_up launch) against
    moe_route_permute + moe_expert_ffn_combine, and the exact oracle."""
    wl = workload_for("decode", T=T)
    flush(f"moe_layer decode T={T}")
    one = _layer_vs_calls(moe, wl)
    exact = oracle.moe_layer(wl.x_bf16, wl.logits, wl.weights, wl.K)
    assert normwise(bf16_np(one["out"]), exact["out"]) <= 2e-2


@pytest.mark.parametrize("cfg", [
    dict(T=8, H=2048, E=1000, K=10, I=512, has_shared=True),   # E > 512: 16 logits per lane
    dict(T=8, H=2048, E=1024, K=32, I=512, has_shared=False),  # the largest E and K
    dict(T=5, H=2048, E=64, K=10, I=512, has_shared=True),
    dict(T=8, H=256, E=4, K=2, I=128, has_shared=True),       # smallest H and I, few groups
    dict(T=7, H=1024, E=16, K=4, I=1024, has_shared=False),
    dict(T=3, H=512, E=16, K=4, I=256, has_shared=True),      # gate_up K split in the calls
    dict(T=3, H=1024, E=32, K=4, I=1024, has_shared=True),    # down + combine in one launch, I = 1024
    dict(T=8, H=512, E=16, K=4, I=256, has_shared=True),      # down + combine with 8 staged rows
    dict(T=1, H=2048, E=512, K=1, I=512, has_shared=False),   # one slot
    dict(T=7, H=4096, E=16, K=4, I=1024, has_shared=False),   # no decode kernels: the calls' path
    dict(T=40, H=512, E=16, K=4, I=256, has_shared=True),     # T > 8: the calls' path
])
def test_layer_one_call_shapes(moe, cfg):
    wl = make_workload("ly", seed=13, **cfg)
    flush(f"moe_layer {cfg}")
    _layer_vs_calls(moe, wl)


def test_layer_one_call_arms_and_gate(moe):
    wl = workload_for("decode", T=8)
    g = torch.from_numpy(np.linspace(-3, 3, wl.T).astype(np.float32)).cuda()
    for act_mode in (0, 1, 2, 3):   # 2 and 3 (per-class arms) take the calls' path
        flush(f"moe_layer arms act_mode={act_mode}")
        _layer_vs_calls(moe, wl, act_mode=act_mode)
    _layer_vs_calls(moe, wl, act_mode=1, gate=g)
    _layer_vs_calls(moe, wl, act_mode=0, gate=g)
    wl2 = workload_for("decode", T=2)   # the gated combine inside the down launch
    g2 = torch.from_numpy(np.array([-1.5, 2.0], dtype=np.float32)).cuda()
    flush("moe_layer gated, down + combine in one launch")
    _layer_vs_calls(moe, wl2, act_mode=0, gate=g2)
    _layer_vs_calls(moe, wl2, act_mode=1, gate=g2)


@pytest.mark.parametrize("I", [512, 256])   # the fused prefill kernel, and the two-launch one
@pytest.mark.parametrize("act_mode", [0, 1, 2, 3])
def test_layer_grouped_path_arms_and_gate(moe, act_mode, I):
    """Batches above 8 tokens: the routing and the activation prep (one arm,
    or two for the per-class arms 2 and 3) share one launch; the layer equals
    the separate calls bit for bit, with and without the shared-expert gate."""
    T = 72
    wl = make_workload("lg", T=T, H=512, E=32, K=4, I=I, has_shared=True, seed=17 + act_mode)
    flush(f"moe_layer grouped path act_mode={act_mode} I={I}")
    _layer_vs_calls(moe, wl, act_mode=act_mode)
    g = torch.from_numpy(np.linspace(-2.5, 2.5, T).astype(np.float32)).cuda()
    _layer_vs_calls(moe, wl, act_mode=act_mode, gate=g)


def test_layer_one_call_ties_and_invalid_rows(moe):
    """All-equal, NaN and -inf logit rows: the layer's routing is the router
    stage's rule in every block, and block 0 publishes it."""
    wl = make_workload("lt", T=4, H=512, E=64, K=6, I=256, has_shared=True, seed=21)
    lg = wl.logits.copy()
    lg[0, :] = 0.0
    lg[1, 5] = np.nan
    lg[2, :] = -np.inf
    lg[3, ::2] = np.inf
    wl.logits = np.ascontiguousarray(lg)
    _layer_vs_calls(moe, wl)


@pytest.mark.parametrize("T", DECODE_TS)
def test_fused_layer_against_oracle(moe, T):
    """moe_layer(fused=True), the one-call layer, through the same gates as the
    unfused layer."""
    wl = workload_for("decode", T=T)
    W = moe.NVFP4Weights.from_bank(wl.weights)
    r = moe.moe_layer(W, x_dev(wl.x_bf16), torch.from_numpy(wl.logits).cuda(), wl.K, fused=True)
    torch.cuda.synchronize()
    exact = oracle.moe_layer(wl.x_bf16, wl.logits, wl.weights, wl.K)
    emul = oracle.moe_layer(wl.x_bf16, wl.logits, wl.weights, wl.K, h_round="bf16",
                            y_round="bf16")
    assert np.array_equal(r["ids"].cpu().numpy(), exact["ids"])
    assert np.array_equal(r["sorted_slot"].cpu().numpy(), exact["sorted_slot"])
    out = bf16_np(r["out"])
    assert normwise(out, emul["out"]) <= 8e-3
    assert normwise(out, exact["out"]) <= 2e-2
