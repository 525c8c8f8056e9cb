"""GPU parity of the expert FFN (A3-A9) and the combine (A10) against the fp64
oracle.

Gates (the reading of "max relative error" taken here: normwise over the whole
output: max|y - y_ref| / max|y_ref|):
  * bf16 path vs the exact fp64 oracle:                    <= 2e-2
  * FP8-activation arm vs the exact fp64 oracle:           <= 6e-2
  * either path vs the oracle that rounds h and the per-slot outputs to bf16
    where the GPU stores bf16 (and quantises x in the FP8 arm): <= 8e-3,
    tight enough to catch a wrong block scale or a dropped term.
Derivation of the bounds: h and y are stored in bf16 (relative rounding
2^-9 each) and the output is rounded once more, so the bf16 path sits near
3 x 2^-9 ~ 6e-3 normwise in the worst element; f32 accumulation over K <= 2048
adds ~1e-6.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu import bf16_np, flush, normwise, setup, x_dev
from oracle.ffn import bf16_bits_to_f64
from workloads import DECODE_TS, make_workload, workload_for

pytestmark = pytest.mark.gpu

GATE_BF16, GATE_FP8, GATE_TIGHT = 2e-2, 6e-2, 8e-3
# act_mode of the C ABI -> the oracle's arm
ARMS = {0: "bf16", 1: "fp8_row", 2: "fp8_routed", 3: "fp8_shared"}


@pytest.fixture(scope="module")
def moe():
    return setup()


def _run(moe, wl, act_mode=0, W=None):
    W = W or moe.NVFP4Weights.from_bank(wl.weights)
    r = moe.moe_layer(W, x_dev(wl.x_bf16), torch.from_numpy(wl.logits).cuda(), wl.K, act_mode)
    torch.cuda.synchronize()
    return r


def _full_check(moe, wl, act_mode=0, tag=""):
    r = _run(moe, wl, act_mode)
    om = ARMS[act_mode]
    exact = oracle.moe_layer(wl.x_bf16, wl.logits, wl.weights, wl.K)
    emul = oracle.moe_layer(wl.x_bf16, wl.logits, wl.weights, wl.K, act_mode=om,
                            h_round="bf16", y_round="bf16")
    # integer stages bit-exact
    assert np.array_equal(r["ids"].cpu().numpy(), exact["ids"])
    assert np.array_equal(r["sorted_slot"].cpu().numpy(), exact["sorted_slot"])
    y = bf16_np(r["y_slots"])
    out = bf16_np(r["out"])
    e_y = normwise(y, emul["y_slots"])
    e_tight = normwise(out, emul["out"])
    e_exact = normwise(out, exact["out"])
    flush(f"{tag} act={om}: y vs emul {e_y:.2e}  out vs emul {e_tight:.2e}  out vs exact {e_exact:.2e}")
    assert e_y <= GATE_TIGHT
    assert e_tight <= GATE_TIGHT
    assert e_exact <= (GATE_FP8 if act_mode else GATE_BF16)
    # combine on the GPU's own per-slot outputs and weights, fp64, within one bf16 rounding
    ref = oracle.combine(y, r["w"].cpu().numpy().astype(np.float64), r["slot_pos"].cpu().numpy(),
                         wl.T, wl.K, wl.has_shared)
    mag = np.max(np.abs(ref), axis=1, keepdims=True)
    assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * mag)
    return r


def test_tiny_layer(moe):
    _full_check(moe, workload_for("tiny"), tag="tiny")


@pytest.mark.parametrize("T", DECODE_TS)
def test_decode_layer_full_size(moe, T):
    _full_check(moe, workload_for("decode", T=T), tag=f"decode T={T}")


@pytest.mark.parametrize("cfg", [
    dict(T=300, H=2048, E=64, K=10, I=512, has_shared=True),     # ragged tiles, H=2048
    dict(T=700, H=256, E=4, K=2, I=128, has_shared=True),        # several 128-row tiles per expert
    dict(T=9, H=512, E=16, K=4, I=256, has_shared=False),        # just above the decode switch
    dict(T=64, H=1024, E=512, K=10, I=384, has_shared=True),     # many empty experts, I % 256 != 0
    dict(T=40, H=4096, E=8, K=2, I=1024, has_shared=True),       # largest H and I: 32 K steps, 4 + 8 N tiles
])
def test_grouped_path_medium(moe, cfg):
    wl = make_workload("m", seed=3, **cfg)
    _full_check(moe, wl, tag=f"grouped {cfg}")


@pytest.mark.parametrize("cfg", [
    dict(T=4, H=256, E=8, K=2, I=128, has_shared=False),
    dict(T=8, H=2048, E=512, K=10, I=512, has_shared=True),
    dict(T=300, H=2048, E=64, K=10, I=512, has_shared=True),
])
def test_fp8_arm(moe, cfg):
    wl = make_workload("f", seed=4, x_kind="student_t", **cfg)
    r = _full_check(moe, wl, act_mode=1, tag=f"fp8 {cfg}")
    # the row quantisation itself is bit-exact: codes and scales sit in the workspace
    W = moe.NVFP4Weights.from_bank(wl.weights)
    _, ws = moe.moe_expert_ffn(W, x_dev(wl.x_bf16), wl.K, r["offsets"], r["sorted_slot"],
                               r["groups"], 1, return_ws=True)
    torch.cuda.synchronize()
    S = wl.T * wl.K + (wl.T if wl.has_shared else 0)
    off = (S * wl.I * 2 + 255) // 256 * 256
    q = ws[off:off + wl.T * wl.H].cpu().numpy().reshape(wl.T, wl.H)
    off2 = off + (wl.T * wl.H + 255) // 256 * 256
    s = ws[off2:off2 + 4 * wl.T].cpu().numpy().view(np.float32)
    qo, so = oracle.rowquant_e4m3(bf16_bits_to_f64(wl.x_bf16).astype(np.float32))
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("act_mode", [0, 1])
@pytest.mark.parametrize("T", [12, 6])   # grouped path; decode path (rows converted in LDS)
def test_zero_rows(moe, T, act_mode):
    wl = make_workload("z", T=T, H=256, E=8, K=2, I=128, has_shared=True, seed=6)
    wl.x_bf16[3] = 0
    wl.x_bf16[T - 1] = 0x8000      # -0.0
    r = _full_check(moe, wl, act_mode=act_mode, tag=f"zero rows T={T} act={act_mode}")
    # a zero token row gives exactly zero from every expert it reaches
    for t in (3, T - 1):
        assert not np.any(bf16_np(r["out"][t]))


# every e4m3 code that is not NaN (0x7F, 0xFF): zeros, subnormals 0x01-0x07,
# normals up to 0x7E = 448, and the same with the sign bit set
ALL_SCALE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _all_codes_bank(wl, seed):
    """Block scales that run through every finite e4m3 code of both signs, each
    code on many blocks (a seeded shuffle of the cycled list)."""
    rng = np.random.default_rng(seed)
    for name in ("gu_scales", "dn_scales"):
        a = getattr(wl.weights, name)
        cyc = np.resize(ALL_SCALE_CODES, a.size)
        setattr(wl.weights, name, rng.permutation(cyc).reshape(a.shape).astype(np.uint8))
    return wl


@pytest.mark.parametrize("act_mode", [0, 1])
@pytest.mark.parametrize("T", [6, 40])   # decode path; grouped path
def test_every_finite_e4m3_block_scale(moe, T, act_mode):
    """Subnormal, large (products up to 6 x 448 = 2688) and negative block
    scales, which the synthetic generator never draws, on both regimes and both
    activation arms, at the tight gate."""
    wl = make_workload("c", T=T, H=256, E=8, K=2, I=128, has_shared=True, seed=13,
                       x_kind="student_t" if act_mode else "normal")
    _all_codes_bank(wl, 13 + T)
    for name in ("gu_scales", "dn_scales"):
        assert set(np.unique(getattr(wl.weights, name)).tolist()) == set(ALL_SCALE_CODES.tolist())
    _full_check(moe, wl, act_mode=act_mode, tag=f"all e4m3 scale codes T={T} act={act_mode}")


def test_fp8_codes_written_when_no_group_is_active(moe):
    """Every id out of range and no shared expert: no group is active, the FFN
    computes nothing, and the row codes and scales in the workspace are still
    the call's row quantisation of x."""
    wl = make_workload("n", T=5, H=512, E=16, K=3, I=256, has_shared=False, seed=14,
                       x_kind="student_t")
    ids = torch.full((wl.T, wl.K), -1, dtype=torch.int32, device="cuda")
    counts, offsets, sorted_slot, slot_pos, groups = moe.moe_permute(ids, wl.E, False)
    W = moe.NVFP4Weights.from_bank(wl.weights)
    _, ws = moe.moe_expert_ffn(W, x_dev(wl.x_bf16), wl.K, offsets, sorted_slot, groups, 1,
                               return_ws=True)
    torch.cuda.synchronize()
    assert int(groups[0]) == 0
    S = wl.T * wl.K
    off = (S * wl.I * 2 + 255) // 256 * 256
    q = ws[off:off + wl.T * wl.H].cpu().numpy().reshape(wl.T, wl.H)
    off2 = off + (wl.T * wl.H + 255) // 256 * 256
    s = ws[off2:off2 + 4 * wl.T].cpu().numpy().view(np.float32)
    qo, so = oracle.rowquant_e4m3(bf16_bits_to_f64(wl.x_bf16).astype(np.float32))
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("cfg", [
    dict(T=3, H=512, E=32, K=4, I=256, has_shared=True),      # decode, 4 chunks per lane
    dict(T=7, H=1024, E=64, K=6, I=1024, has_shared=True),    # decode, 8 chunks, down with 8 chunks
    dict(T=8, H=1024, E=16, K=8, I=128, has_shared=False),    # decode, one down chunk
    dict(T=2, H=4096, E=8, K=2, I=128, has_shared=True),      # T <= 8 with no decode variant: grouped path
    dict(T=5, H=1024, E=16, K=3, I=384, has_shared=True),     # I / 128 = 3: grouped path at T <= 8
    dict(T=8, H=2048, E=16, K=4, I=1024, has_shared=True),    # decode at its largest H and I
])
def test_small_T_shapes(moe, cfg):
    _full_check(moe, make_workload("q", seed=9, **cfg), tag=f"small T {cfg}")
    _full_check(moe, make_workload("q", seed=10, x_kind="student_t", **cfg), act_mode=1,
                tag=f"small T fp8 {cfg}")


@pytest.mark.parametrize("act_mode", [0, 1])
def test_decode_group_of_more_than_16_rows(moe, act_mode):
    """Caller-supplied ids that repeat one expert (not something the router
    produces): at T=8, K=10, 72 slots go to expert 3, so the decode path's down
    kernel runs the group in five passes of up to 16 rows (the last one partial)
    and gate_up's epilogue reads positions past 64 from sorted_slot.  Every
    per-slot output is checked against the oracle."""
    wl = make_workload("r", T=8, H=1024, E=16, K=10, I=256, has_shared=True, seed=12,
                       x_kind="student_t" if act_mode else "normal")
    ids = np.full((wl.T, wl.K), 3, dtype=np.int32)
    ids[:, 9] = np.arange(wl.T) % 5 + 6
    counts, offsets, sorted_slot, slot_pos, groups = moe.moe_permute(
        torch.from_numpy(ids).cuda(), wl.E, wl.has_shared)
    assert int(counts[3]) == 72
    W = moe.NVFP4Weights.from_bank(wl.weights)
    y = moe.moe_expert_ffn(W, x_dev(wl.x_bf16), wl.K, offsets, sorted_slot, groups, act_mode)
    torch.cuda.synchronize()
    x = bf16_bits_to_f64(wl.x_bf16)
    xin = oracle.rowquant_dequant(x.astype(np.float32)) if act_mode else x
    ref = oracle.ffn.expert_outputs(xin, wl.weights, wl.T, wl.K, offsets.cpu().numpy(),
                                    sorted_slot.cpu().numpy(), h_round="bf16")
    e = normwise(bf16_np(y), ref)
    flush(f"group of 72 rows act={act_mode}: y vs emul {e:.2e}")
    assert e <= GATE_TIGHT


@pytest.mark.parametrize("cfg", [
    dict(T=5, H=256, E=8, K=1, I=128, has_shared=False),
    dict(T=20, H=256, E=8, K=8, I=128, has_shared=False),
    dict(T=1, H=256, E=1, K=1, I=128, has_shared=True),
    dict(T=33, H=256, E=8, K=1, I=128, has_shared=True),
])
def test_degenerate_routing(moe, cfg):
    _full_check(moe, make_workload("d", seed=7, **cfg), tag=f"degenerate {cfg}")


def test_scale2_is_applied(moe):
    wl = make_workload("s", T=40, H=256, E=8, K=2, I=128, has_shared=True, seed=8)
    rng = np.random.default_rng(0)
    wl.weights.scale2[:] = rng.uniform(0.25, 3.0, wl.weights.scale2.shape).astype(np.float32)
    _full_check(moe, wl, tag="scale2")
    wl2 = make_workload("s", T=6, H=256, E=8, K=2, I=128, has_shared=True, seed=8)
    wl2.weights.scale2[:] = wl.weights.scale2
    _full_check(moe, wl2, tag="scale2 decode")


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_token_permutation_is_bitwise_equivariant(moe, name):
    wl = workload_for(name, T=8 if name == "decode" else 512)
    W = moe.NVFP4Weights.from_bank(wl.weights)
    a = _run(moe, wl, W=W)["out"]
    p = np.random.default_rng(1).permutation(wl.T)
    wl.x_bf16 = np.ascontiguousarray(wl.x_bf16[p])
    wl.logits = np.ascontiguousarray(wl.logits[p])
    b = _run(moe, wl, W=W)["out"]
    assert torch.equal(a[torch.from_numpy(p).cuda()].view(torch.int16), b.view(torch.int16))


def test_repeated_layer_calls_are_bitwise_identical(moe):
    wl = workload_for("prefill", T=1024)
    W = moe.NVFP4Weights.from_bank(wl.weights)
    a = _run(moe, wl, W=W)
    b = _run(moe, wl, W=W)
    for k in ("y_slots", "out"):
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))


def _whole_groups(counts, E, name):
    """Groups whose every row is recomputed by the oracle at full size: the
    shared group, the largest routed group, and one routed group for each size
    of a last partial 128-row tile (1-32, 33-64, 65-96 and 97-127 rows past the
    last full tile), so every tile shape of the grouped kernel is covered."""
    routed = counts[:E]
    pick = {E, int(np.argmax(routed))}
    rem = routed % 128
    for lo, hi in ((1, 32), (33, 64), (65, 96), (97, 127)):
        cand = np.nonzero((rem >= lo) & (rem <= hi))[0]
        if cand.size:
            pick.add(int(cand[0]))
    return sorted(pick)


def _sampled_check(moe, name, act_mode=0, n_tok=6):
    """Full-size run.  The oracle recomputes (1) every row of a few whole groups
    (_whole_groups) and (2) a sample of tokens: all their routed experts and the
    shared expert, per slot and after the combine."""
    wl = workload_for(name)
    flush(f"sampled {name} T={wl.T} act={act_mode}")
    r = _run(moe, wl, act_mode)
    ids = r["ids"].cpu().numpy()
    ids_o, w_o = oracle.route_topk(wl.logits, wl.K)
    assert np.array_equal(ids, ids_o)
    counts_o, offsets_o, sorted_o, slot_pos_o = oracle.permute(ids_o, wl.E, wl.has_shared)
    for got, want in zip((r["counts"], r["offsets"], r["sorted_slot"], r["slot_pos"]),
                         (counts_o, offsets_o, sorted_o, slot_pos_o)):
        assert np.array_equal(got.cpu().numpy(), want)
    slot_pos = r["slot_pos"].cpu().numpy()
    y_gpu = r["y_slots"]
    x_all = bf16_bits_to_f64(wl.x_bf16)
    xin_all = oracle.rowquant_dequant(x_all.astype(np.float32)) if act_mode else x_all

    # (1) whole groups
    groups = _whole_groups(counts_o, wl.E, name)
    for g in groups:
        a, b = int(offsets_o[g]), int(offsets_o[g + 1])
        # offsets that put group g alone at positions [0, b - a), so the
        # oracle's output holds only this group's rows
        offs = np.zeros_like(offsets_o)
        offs[g + 1:] = b - a
        ref = oracle.ffn.expert_outputs(xin_all, wl.weights, wl.T, wl.K, offs, sorted_o[a:b],
                                        h_round="bf16", groups=[g])
        got = bf16_np(y_gpu[a:b])
        e = normwise(got, ref)
        flush(f"  whole group {g}: {b - a} rows ({(b - a) % 128} in the last tile)  "
              f"y vs emul {e:.2e}")
        assert e <= GATE_TIGHT

    # (2) sampled tokens
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, n_tok, replace=False)]))
    cache = {}

    def ffn(e, rows, h_round):
        if e not in cache:
            cache[e] = oracle.ffn.dequant_expert(wl.weights, e)
        return oracle.expert_ffn(rows, *cache[e], h_round=h_round)

    out_gpu = bf16_np(r["out"][torch.from_numpy(toks).cuda()])
    worst_y = 0.0
    out_ref = np.zeros_like(out_gpu)
    for i, t in enumerate(toks):
        xin = xin_all[t:t + 1]
        for k in range(wl.K):
            e = int(ids[t, k])
            yk = ffn(e, xin, "none")[0]
            ye = ffn(e, xin, "bf16")[0]
            yg = bf16_np(y_gpu[int(slot_pos[t * wl.K + k])])
            worst_y = max(worst_y, normwise(yg, ye))
            out_ref[i] += w_o[t, k] * yk
        out_ref[i] += ffn(wl.E, xin, "none")[0]    # the shared expert, same input arm
    e_out = normwise(out_gpu, out_ref)
    flush(f"  sampled {len(toks)} tokens: worst y vs emul {worst_y:.2e}  out vs oracle {e_out:.2e}")
    assert worst_y <= GATE_TIGHT
    assert e_out <= (GATE_TIGHT if not act_mode else GATE_FP8)
    return groups


def test_prefill_full_size_sampled(moe):
    _sampled_check(moe, "prefill")


def test_long_prefill_full_size_sampled(moe):
    _sampled_check(moe, "long_prefill")


def test_fp8_arm_full_size_sampled(moe):
    _sampled_check(moe, "fp8_arm", act_mode=1)
    _sampled_check(moe, "fp8_arm", act_mode=0)


@pytest.mark.parametrize("act_mode", [2, 3])
@pytest.mark.parametrize("cfg", [
    dict(name="decode", T=8, H=2048, E=512, K=10, I=512, has_shared=True),   # decode GEMV
    dict(name="decode1", T=1, H=2048, E=512, K=10, I=512, has_shared=True),
    dict(name="fused", T=300, H=2048, E=64, K=10, I=512, has_shared=True),   # fused prefill kernel
    dict(name="twolaunch", T=700, H=256, E=4, K=2, I=128, has_shared=True),  # two-launch prefill
    dict(name="noshared", T=40, H=512, E=16, K=4, I=256, has_shared=False),
])
def test_per_class_activation_arms(moe, cfg, act_mode):
    """Routed e4m3 with the shared expert on bf16 (the A/B table's arm S), and
    the mirror, against the oracle's arm, on every FFN path."""
    cfg = dict(cfg)
    name = cfg.pop("name")
    wl = make_workload("arm", seed=21, x_kind="student_t", **cfg)
    _full_check(moe, wl, act_mode=act_mode, tag=f"arm {act_mode} {name}")
