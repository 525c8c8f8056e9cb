"""The allocation-free expert FFN (moe_expert_ffn_noalloc) against the
caller-workspace entry point (moe_expert_ffn): the same kernels on the same
inputs, so the outputs must be bitwise identical.  Two calls in a row on the
library's one fixed workspace, the second smaller than the first (stale
contents from the first call must not leak into the second), in both
activation arms, on the grouped and the decode regime; sizes beyond the fixed
workspace are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from _gpu import bf16_np, flush, normwise, setup, x_dev
from oracle.ffn import bf16_bits_to_f64
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    return setup()


def _inputs(moe, wl):
    W = moe.NVFP4Weights.from_bank(wl.weights)
    ids, w = moe.moe_route_topk(torch.from_numpy(wl.logits).cuda(), wl.K)
    perm = moe.moe_permute(ids, wl.E, wl.has_shared)
    return W, x_dev(wl.x_bf16), perm


@pytest.mark.parametrize("act_mode", [0, 1])
def test_noalloc_matches_workspace_entry_point(moe, act_mode):
    xk = "student_t" if act_mode else "normal"
    big = make_workload("a", T=1500, H=2048, E=64, K=10, I=512, has_shared=True, seed=21, x_kind=xk)
    small = make_workload("b", T=6, H=2048, E=64, K=10, I=512, has_shared=True, seed=22, x_kind=xk)
    for wl, tag in ((big, "first call, grouped path T=1500"), (small, "second call, decode path T=6")):
        flush(f"noalloc act={act_mode}: {tag}")
        W, x, (counts, offsets, sorted_slot, slot_pos, groups) = _inputs(moe, wl)
        S = wl.T * wl.K + wl.T
        y_ws = moe.moe_expert_ffn(W, x, wl.K, offsets, sorted_slot, groups, act_mode)
        y_na = torch.full((S, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_expert_ffn_noalloc(W, x, wl.K, offsets, sorted_slot, groups, act_mode, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16)), tag
        # and the pair sits at the oracle's tight gate (sampled groups)
        off = offsets.cpu().numpy()
        ss = sorted_slot.cpu().numpy()
        xin = bf16_bits_to_f64(wl.x_bf16)
        if act_mode:
            xin = oracle.rowquant_dequant(xin.astype(np.float32))
        g = int(np.argmax(np.diff(off)[:wl.E]))
        a, b = int(off[g]), int(off[g + 1])
        offs = np.zeros_like(off)
        offs[g + 1:] = b - a
        ref = oracle.ffn.expert_outputs(xin, wl.weights, wl.T, wl.K, offs, ss[a:b],
                                        h_round="bf16", groups=[g])
        e = normwise(bf16_np(y_na[a:b]), ref)
        flush(f"  group {g} ({b - a} rows) y vs emul {e:.2e}")
        assert e <= 8e-3


def test_noalloc_refuses_sizes_beyond_its_workspace(moe):
    from bit_block_quantized_nvfp4_amd import _lib as L

    lib = L.lib()
    one = ctypes.c_void_p(16)
    W = L.MoeNvfp4Weights(16, 16, 16, 16, 16, 512, 2048, 512, 1)
    need = lib.moe_workspace_bytes(L.MOE_OP_EXPERT_FFN, 2184, 512, 10, 2048, 512, 1, 0)
    assert need > L.MOE_NOALLOC_WS_BYTES
    rc = lib.moe_expert_ffn_noalloc(ctypes.byref(W), one, 2184, 10, one, one, one, 0, one, None)
    assert rc == L.MOE_EWORKSPACE
    assert b"fixed" in lib.moe_last_error()
    assert lib.moe_workspace_bytes(L.MOE_OP_EXPERT_FFN, 2183, 512, 10, 2048, 512, 1, 0) <= L.MOE_NOALLOC_WS_BYTES
