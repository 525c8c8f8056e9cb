"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (no GPU needed: argument errors return before any HIP
call)."""
import ctypes

import pytest

from _libutil import declared_functions, ensure_built


@pytest.fixture(scope="module")
def lib():
    ensure_built()
    from bit_block_quantized_nvfp4_amd import _lib

    return _lib.lib()


def test_header_declares_the_four_layer_calls():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_init",
              "moe_last_error", "moe_workspace_bytes", "moe_router_topk", "moe_combine_gated", "moe_route_permute",
              "moe_expert_ffn_combine", "moe_layer"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(lib._name)
    for n in declared_functions():
        assert hasattr(raw, n), n


def test_argument_errors_are_reported_without_a_gpu(lib):
    from bit_block_quantized_nvfp4_amd import _lib as L

    P = ctypes.c_void_p
    one = P(16)
    assert lib.moe_route_topk(None, 4, 8, 2, one, one, None) == L.MOE_EINVAL
    assert b"null" in lib.moe_last_error()
    assert lib.moe_route_topk(one, 4, 8, 9, one, one, None) == L.MOE_EINVAL     # K > E
    assert lib.moe_route_topk(one, 4, 2048, 2, one, one, None) == L.MOE_EINVAL  # E > 1024
    assert lib.moe_route_topk(one, 4, 64, 33, one, one, None) == L.MOE_EINVAL   # K > 32
    assert lib.moe_route_topk(one, 0, 8, 2, one, one, None) == L.MOE_EINVAL     # T < 1
    assert lib.moe_permute(one, 4, 8, 2, 2, one, one, one, one, one, None, 0, None) == L.MOE_EINVAL
    assert lib.moe_permute(one, 4, 8, 2, 0, one, one, one, one, None, None, 0, None) == L.MOE_EINVAL
    # a large permute needs a workspace
    assert lib.moe_permute(one, 4096, 512, 10, 1, one, one, one, one, one, None, 0, None) == L.MOE_EWORKSPACE
    W = L.MoeNvfp4Weights(16, 16, 16, 16, 16, 8, 256, 128, 0)
    ffn = lib.moe_expert_ffn
    assert ffn(ctypes.byref(W), one, 4, 2, one, one, one, 7, one, one, 1 << 20, None) == L.MOE_EUNSUPPORTED
    bad = L.MoeNvfp4Weights(16, 16, 16, 16, 16, 8, 200, 128, 0)   # H not a multiple of 256
    assert ffn(ctypes.byref(bad), one, 4, 2, one, one, one, 0, one, one, 1 << 20, None) == L.MOE_EINVAL
    assert ffn(ctypes.byref(W), one, 4, 2, one, one, one, 0, one, one, 16, None) == L.MOE_EWORKSPACE
    assert ffn(ctypes.byref(W), one, 4, 2, one, one, None, 0, one, one, 1 << 20, None) == L.MOE_EINVAL
    nullw = L.MoeNvfp4Weights(0, 16, 16, 16, 16, 8, 256, 128, 0)
    assert ffn(ctypes.byref(nullw), one, 4, 2, one, one, one, 0, one, one, 1 << 20, None) == L.MOE_EINVAL
    assert lib.moe_combine(one, one, one, 4, 2, 12, 0, one, None) == L.MOE_EINVAL  # H % 8
    assert lib.moe_combine(one, one, None, 4, 2, 16, 0, one, None) == L.MOE_EINVAL
    cg = lib.moe_combine_gated
    assert cg(one, one, one, None, 4, 2, 16, one, None) == L.MOE_EINVAL       # no gate
    assert cg(one, one, one, one, 4, 2, 12, one, None) == L.MOE_EINVAL        # H % 8
    rp = lib.moe_route_permute
    assert rp(None, 4, 8, 2, 0, one, one, one, one, one, one, one, None, 0, None) == L.MOE_EINVAL
    assert rp(one, 4, 8, 9, 0, one, one, one, one, one, one, one, None, 0, None) == L.MOE_EINVAL  # K > E
    assert rp(one, 4096, 512, 10, 1, one, one, one, one, one, one, one, None, 0, None) == L.MOE_EWORKSPACE
    fc = lib.moe_expert_ffn_combine
    Ws = L.MoeNvfp4Weights(16, 16, 16, 16, 16, 8, 256, 128, 1)
    assert fc(ctypes.byref(Ws), one, 4, 2, one, one, one, 0, None, one, None, one, one, one, 1 << 20,
              None) == L.MOE_EINVAL                                                       # no w
    assert fc(ctypes.byref(W), one, 4, 2, one, one, one, 0, one, one, one, one, one, one, 1 << 20,
              None) == L.MOE_EINVAL                                                       # gate, no shared
    assert fc(ctypes.byref(Ws), one, 4, 2, one, one, one, 5, one, one, None, one, one, one, 1 << 20,
              None) == L.MOE_EUNSUPPORTED
    need = lib.moe_workspace_bytes(L.MOE_OP_EXPERT_FFN_COMBINE, 4, 8, 2, 256, 128, 1, 0)
    assert need >= lib.moe_workspace_bytes(L.MOE_OP_EXPERT_FFN, 4, 8, 2, 256, 128, 1, 0) > 0
    assert fc(ctypes.byref(Ws), one, 4, 2, one, one, one, 0, one, one, None, one, one, one, need - 1,
              None) == L.MOE_EWORKSPACE
    ly = lib.moe_layer
    nl = lib.moe_workspace_bytes(L.MOE_OP_LAYER, 4, 8, 2, 256, 128, 1, 0)
    assert nl >= need
    assert ly(ctypes.byref(Ws), None, one, 4, 2, 0, None, one, one, one, one, one, one, one, one,
              one, one, nl, None) == L.MOE_EINVAL                                         # no logits
    assert ly(ctypes.byref(Ws), one, one, 4, 2, 7, None, one, one, one, one, one, one, one, one,
              one, one, nl, None) == L.MOE_EUNSUPPORTED                                   # act_mode
    assert ly(ctypes.byref(W), one, one, 4, 2, 0, one, one, one, one, one, one, one, one, one,
              one, one, nl, None) == L.MOE_EINVAL                                         # gate, no shared
    assert ly(ctypes.byref(Ws), one, one, 4, 9, 0, None, one, one, one, one, one, one, one, one,
              one, one, nl, None) == L.MOE_EINVAL                                         # K > E
    assert ly(ctypes.byref(Ws), one, one, 4, 2, 0, None, one, one, one, one, one, one, one, one,
              one, one, nl - 1, None) == L.MOE_EWORKSPACE
    rt = lib.moe_router_topk
    R = L.MoeNvfp4Router(16, 16, 1.0, 64, 512, 1)
    assert rt(ctypes.byref(R), one, 4, 2, one, one, one, None, None) == L.MOE_EINVAL   # gate row, no gate
    assert rt(ctypes.byref(R), one, 4, 65, one, one, one, one, None) == L.MOE_EINVAL   # K > E
    assert rt(ctypes.byref(R), one, 4, 2, one, one, None, one, None) == L.MOE_EINVAL   # no logits
    Rh = L.MoeNvfp4Router(16, 16, 1.0, 64, 300, 0)                                   # H % 256
    assert rt(ctypes.byref(Rh), one, 4, 2, one, one, one, None, None) == L.MOE_EINVAL
    Rb = L.MoeNvfp4Router(16, 16, 1.0, 64, 16384, 0)                                 # H > 8192
    assert rt(ctypes.byref(Rb), one, 4, 2, one, one, one, None, None) == L.MOE_EINVAL
    Rn = L.MoeNvfp4Router(0, 16, 1.0, 64, 512, 0)                                    # null codes
    assert rt(ctypes.byref(Rn), one, 4, 2, one, one, one, None, None) == L.MOE_EINVAL
    Rg = L.MoeNvfp4Router(16, 16, 1.0, 64, 512, 2)                                   # has_gate 2
    assert rt(ctypes.byref(Rg), one, 4, 2, one, one, one, one, None) == L.MOE_EINVAL


def test_workspace_sizes(lib):
    from bit_block_quantized_nvfp4_amd import _lib as L

    ws = lib.moe_workspace_bytes
    # the decode permutation runs in one workgroup without a workspace
    assert ws(L.MOE_OP_PERMUTE, 8, 512, 10, 0, 0, 1, 0) == 0
    assert ws(L.MOE_OP_PERMUTE, 4096, 512, 10, 0, 0, 1, 0) > 0
    S = 4096 * 10 + 4096
    bf = ws(L.MOE_OP_EXPERT_FFN, 4096, 512, 10, 2048, 512, 1, L.MOE_ACT_BF16)
    fp8 = ws(L.MOE_OP_EXPERT_FFN, 4096, 512, 10, 2048, 512, 1, L.MOE_ACT_FP8_ROW)
    assert bf >= S * 512 * 2 and fp8 >= bf + 4096 * 2048 + 4096 * 4
    assert ws(L.MOE_OP_EXPERT_FFN, 4096, 512, 10, 2048, 512, 1, 9) == 0
    # the layer's workspace serves the permutation, then the FFN + combine
    for T in (8, 4096):
        lay = ws(L.MOE_OP_LAYER, T, 512, 10, 2048, 512, 1, L.MOE_ACT_BF16)
        assert lay >= ws(L.MOE_OP_PERMUTE, T, 512, 10, 0, 0, 1, 0)
        assert lay >= ws(L.MOE_OP_EXPERT_FFN_COMBINE, T, 512, 10, 2048, 512, 1, L.MOE_ACT_BF16)
    assert ws(99, 4, 8, 2, 256, 128, 0, 0) == 0
