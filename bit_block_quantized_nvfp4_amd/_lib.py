"""ctypes loader for libmoe_nvfp4.so (the HIP library built from csrc/).

There is no fallback: if the library is missing or cannot be loaded, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_nvfp4.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EHIP = -3
MOE_EWORKSPACE = -4
MOE_ACT_BF16 = 0
MOE_ACT_FP8_ROW = 1
MOE_ACT_FP8_ROUTED = 2
MOE_ACT_FP8_SHARED = 3
MOE_OP_PERMUTE = 1
MOE_OP_EXPERT_FFN = 2
MOE_OP_EXPERT_FFN_COMBINE = 3
MOE_OP_LAYER = 4
MOE_NOALLOC_WS_BYTES = 32 << 20


class MoeNvfp4Weights(ctypes.Structure):
    _fields_ = [
        ("gu_codes", ctypes.c_void_p),
        ("gu_scales", ctypes.c_void_p),
        ("dn_codes", ctypes.c_void_p),
        ("dn_scales", ctypes.c_void_p),
        ("scale2", ctypes.c_void_p),
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("has_shared", ctypes.c_int32),
    ]


class MoeNvfp4Router(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("scale2", ctypes.c_float),
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("has_gate", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"moe_nvfp4 status {status}: {msg}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_init": (_I, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "moe_route_topk": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_permute": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn": (_I, [ctypes.POINTER(MoeNvfp4Weights), _P, _I, _I, _P, _P, _P, _I, _P, _P, _SZ, _P]),
    "moe_expert_ffn_noalloc": (_I, [ctypes.POINTER(MoeNvfp4Weights), _P, _I, _I, _P, _P, _P, _I,
                                    _P, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_route_permute": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn_combine": (_I, [ctypes.POINTER(MoeNvfp4Weights), _P, _I, _I, _P, _P, _P, _I,
                                    _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_combine_gated": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_layer": (_I, [ctypes.POINTER(MoeNvfp4Weights), _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                       _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_router_topk": (_I, [ctypes.POINTER(MoeNvfp4Router), _P, _I, _I, _P, _P, _P, _P, _P]),
    "moe_timing_enable": (_I, [_I]),
    "moe_timing_reset": (_I, []),
    "moe_timing_read": (_I, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_I),
                             ctypes.POINTER(ctypes.c_double), _I, ctypes.POINTER(_I)]),
}


def lib():
    """Load (once) and return the ctypes handle of libmoe_nvfp4.so."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run bit_block_quantized_nvfp4_amd/build.py "
                "(hipcc --offload-arch=gfx950)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def check(status: int) -> int:
    if status < 0:
        raise MoeError(status, lib().moe_last_error().decode(errors="replace"))
    return status
