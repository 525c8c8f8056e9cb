"""Python binding of the C ABI (include/moe_nvfp4.h): argument marshalling only.

Every function takes and returns torch tensors on the current HIP device and
enqueues the library's kernels on torch's current stream.  Outputs (and, unless
given, workspaces) are allocated with torch; all arithmetic runs in the HIP
kernels of libmoe_nvfp4.so.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (MOE_ACT_BF16, MOE_ACT_FP8_ROUTED, MOE_ACT_FP8_ROW, MOE_ACT_FP8_SHARED,
                   MOE_OP_EXPERT_FFN, MOE_OP_EXPERT_FFN_COMBINE, MOE_OP_LAYER, MOE_OP_PERMUTE,
                   check)

__all__ = [
    "NVFP4Weights", "moe_init", "moe_route_topk", "moe_permute", "moe_expert_ffn",
    "moe_combine", "moe_layer", "workspace_bytes", "moe_expert_ffn_noalloc", "MOE_ACT_BF16", "MOE_ACT_FP8_ROW",
    "NVFP4Router", "moe_router_topk", "moe_combine_gated", "moe_route_permute",
    "moe_expert_ffn_combine", "MOE_ACT_FP8_ROUTED", "MOE_ACT_FP8_SHARED",
]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, dtype, shape=None, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass
class NVFP4Weights:
    """A device-resident NVFP4 expert bank in the layout of moe_nvfp4_weights."""
    gu_codes: torch.Tensor   # uint8 [E', 2I, H/2]
    gu_scales: torch.Tensor  # uint8 [E', 2I, H/16]
    dn_codes: torch.Tensor   # uint8 [E', H, I/2]
    dn_scales: torch.Tensor  # uint8 [E', H, I/16]
    scale2: torch.Tensor     # float32 [E', 3]
    E: int
    H: int
    I: int
    has_shared: bool

    @classmethod
    def from_bank(cls, bank, device="cuda") -> "NVFP4Weights":
        def up(a):
            return torch.from_numpy(a).to(device)
        return cls(up(bank.gu_codes), up(bank.gu_scales), up(bank.dn_codes), up(bank.dn_scales),
                   up(bank.scale2), bank.E, bank.H, bank.I, bool(bank.has_shared))

    def struct(self) -> _lib.MoeNvfp4Weights:
        G, H, I = self.E + int(self.has_shared), self.H, self.I
        _need(self.gu_codes, torch.uint8, (G, 2 * I, H // 2), "gu_codes")
        _need(self.gu_scales, torch.uint8, (G, 2 * I, H // 16), "gu_scales")
        _need(self.dn_codes, torch.uint8, (G, H, I // 2), "dn_codes")
        _need(self.dn_scales, torch.uint8, (G, H, I // 16), "dn_scales")
        _need(self.scale2, torch.float32, (G, 3), "scale2")
        return _lib.MoeNvfp4Weights(self.gu_codes.data_ptr(), self.gu_scales.data_ptr(),
                                    self.dn_codes.data_ptr(), self.dn_scales.data_ptr(),
                                    self.scale2.data_ptr(), self.E, H, I, int(self.has_shared))


@dataclass
class NVFP4Router:
    """A device-resident NVFP4 router matrix in the layout of moe_nvfp4_router:
    E expert rows, plus the shared-expert gate row at index E when has_gate."""
    codes: torch.Tensor   # uint8 [E + has_gate, H/2]
    scales: torch.Tensor  # uint8 [E + has_gate, H/16]
    scale2: float
    E: int
    H: int
    has_gate: bool

    @classmethod
    def from_bank(cls, rb, device="cuda") -> "NVFP4Router":
        return cls(torch.from_numpy(rb.codes).to(device), torch.from_numpy(rb.scales).to(device),
                   float(rb.scale2), rb.E, rb.H, bool(rb.has_gate))

    def struct(self) -> _lib.MoeNvfp4Router:
        R = self.E + int(self.has_gate)
        _need(self.codes, torch.uint8, (R, self.H // 2), "router codes")
        _need(self.scales, torch.uint8, (R, self.H // 16), "router scales")
        return _lib.MoeNvfp4Router(self.codes.data_ptr(), self.scales.data_ptr(), self.scale2,
                                   self.E, self.H, int(self.has_gate))


def moe_init() -> None:
    check(_lib.lib().moe_init())


def workspace_bytes(op: int, T: int, E: int, K: int, H: int = 0, I: int = 0,
                    has_shared: bool = False, act_mode: int = MOE_ACT_BF16) -> int:
    return int(_lib.lib().moe_workspace_bytes(op, T, E, K, H, I, int(has_shared), act_mode))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def moe_route_topk(logits: torch.Tensor, K: int, ids: Optional[torch.Tensor] = None,
                   w: Optional[torch.Tensor] = None):
    _need(logits, torch.float32, name="logits")
    T, E = logits.shape
    ids = torch.empty((T, K), dtype=torch.int32, device=logits.device) if ids is None else ids
    w = torch.empty((T, K), dtype=torch.float32, device=logits.device) if w is None else w
    _need(ids, torch.int32, (T, K), "ids")
    _need(w, torch.float32, (T, K), "w")
    check(_lib.lib().moe_route_topk(_ptr(logits), T, E, K, _ptr(ids), _ptr(w), _stream()))
    return ids, w


def moe_router_topk(R: NVFP4Router, x: torch.Tensor, K: int,
                    ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                    logits: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None):
    """Router GEMM + top-K.  Returns (ids, w, logits, gate logits or None)."""
    _need(x, torch.bfloat16, name="x")
    T, H = x.shape
    if H != R.H:
        raise ValueError("x width does not match the router matrix")
    dev = x.device
    ids = torch.empty((T, K), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, K), dtype=torch.float32, device=dev) if w is None else w
    _need(ids, torch.int32, (T, K), "ids")
    _need(w, torch.float32, (T, K), "w")
    logits = torch.empty((T, R.E), dtype=torch.float32, device=dev) if logits is None else logits
    _need(logits, torch.float32, (T, R.E), "logits")
    if R.has_gate and gate is None:
        gate = torch.empty((T,), dtype=torch.float32, device=dev)
    if gate is not None:
        _need(gate, torch.float32, (T,), "gate")
    st = R.struct()
    check(_lib.lib().moe_router_topk(ctypes.byref(st), _ptr(x), T, K, _ptr(ids), _ptr(w),
                                     _ptr(logits), _ptr(gate), _stream()))
    return ids, w, logits, (gate if R.has_gate else None)


def moe_permute(ids: torch.Tensor, E: int, has_shared: bool, ws: Optional[torch.Tensor] = None,
                out=None):
    _need(ids, torch.int32, name="ids")
    T, K = ids.shape
    G = E + int(has_shared)
    dev = ids.device
    if out is None:
        out = (torch.empty(G, dtype=torch.int32, device=dev),
               torch.empty(G + 1, dtype=torch.int32, device=dev),
               torch.empty(T * K + (T if has_shared else 0), dtype=torch.int32, device=dev),
               torch.empty(T * K + (T if has_shared else 0), dtype=torch.int32, device=dev),
               torch.empty(G + 1, dtype=torch.int32, device=dev))
    counts, offsets, sorted_slot, slot_pos, groups = out
    nb = workspace_bytes(MOE_OP_PERMUTE, T, E, K, 0, 0, has_shared)
    ws = _workspace(nb, dev, ws)
    check(_lib.lib().moe_permute(_ptr(ids), T, E, K, int(has_shared), _ptr(counts), _ptr(offsets),
                                 _ptr(sorted_slot), _ptr(slot_pos), _ptr(groups), _ptr(ws), nb,
                                 _stream()))
    return counts, offsets, sorted_slot, slot_pos, groups


def moe_route_permute(logits: torch.Tensor, K: int, has_shared: bool,
                      ws: Optional[torch.Tensor] = None, out=None):
    """moe_route_topk + moe_permute (one kernel for small batches).
    Returns (ids, w, counts, offsets, sorted_slot, slot_pos, groups)."""
    _need(logits, torch.float32, name="logits")
    T, E = logits.shape
    G = E + int(has_shared)
    S = T * K + (T if has_shared else 0)
    dev = logits.device
    i32 = torch.int32
    if out is None:
        out = (torch.empty((T, K), dtype=i32, device=dev),
               torch.empty((T, K), dtype=torch.float32, device=dev),
               torch.empty(G, dtype=i32, device=dev), torch.empty(G + 1, dtype=i32, device=dev),
               torch.empty(S, dtype=i32, device=dev), torch.empty(S, dtype=i32, device=dev),
               torch.empty(G + 1, dtype=i32, device=dev))
    ids, w, counts, offsets, sorted_slot, slot_pos, groups = out
    _need(ids, i32, (T, K), "ids")
    _need(w, torch.float32, (T, K), "w")
    nb = workspace_bytes(MOE_OP_PERMUTE, T, E, K, 0, 0, has_shared)
    ws = _workspace(nb, dev, ws)
    check(_lib.lib().moe_route_permute(_ptr(logits), T, E, K, int(has_shared), _ptr(ids), _ptr(w),
                                       _ptr(counts), _ptr(offsets), _ptr(sorted_slot),
                                       _ptr(slot_pos), _ptr(groups), _ptr(ws), nb, _stream()))
    return ids, w, counts, offsets, sorted_slot, slot_pos, groups


def moe_expert_ffn_combine(W: NVFP4Weights, x: torch.Tensor, K: int, offsets: torch.Tensor,
                           sorted_slot: torch.Tensor, groups: torch.Tensor, w: torch.Tensor,
                           slot_pos: torch.Tensor, act_mode: int = MOE_ACT_BF16,
                           gate: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                           y_slots: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None):
    """moe_expert_ffn followed by the combine, one call.  Returns (y_slots, out)."""
    _need(x, torch.bfloat16, name="x")
    T, H = x.shape
    if H != W.H:
        raise ValueError("x width does not match the weight bank")
    S = T * K + (T if W.has_shared else 0)
    dev = x.device
    y_slots = torch.empty((S, H), dtype=torch.bfloat16, device=dev) if y_slots is None else y_slots
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(y_slots, torch.bfloat16, (S, H), "y_slots")
    _need(out, torch.bfloat16, (T, H), "out")
    _need(w, torch.float32, (T, K), "w")
    _need(slot_pos, torch.int32, (S,), "slot_pos")
    if gate is not None:
        _need(gate, torch.float32, (T,), "gate")
    nb = workspace_bytes(MOE_OP_EXPERT_FFN_COMBINE, T, W.E, K, H, W.I, W.has_shared, act_mode)
    ws = _workspace(nb, dev, ws)
    st = W.struct()
    check(_lib.lib().moe_expert_ffn_combine(ctypes.byref(st), _ptr(x), T, K, _ptr(offsets),
                                            _ptr(sorted_slot), _ptr(groups), act_mode, _ptr(w),
                                            _ptr(slot_pos), _ptr(gate), _ptr(y_slots), _ptr(out),
                                            _ptr(ws), nb, _stream()))
    return y_slots, out


def moe_expert_ffn(W: NVFP4Weights, x: torch.Tensor, K: int, offsets: torch.Tensor,
                   sorted_slot: torch.Tensor, groups: torch.Tensor, act_mode: int = MOE_ACT_BF16,
                   ws: Optional[torch.Tensor] = None, y_slots: Optional[torch.Tensor] = None,
                   return_ws: bool = False):
    _need(x, torch.bfloat16, name="x")
    T, H = x.shape
    if H != W.H:
        raise ValueError("x width does not match the weight bank")
    S = T * K + (T if W.has_shared else 0)
    dev = x.device
    y_slots = torch.empty((S, H), dtype=torch.bfloat16, device=dev) if y_slots is None else y_slots
    _need(y_slots, torch.bfloat16, (S, H), "y_slots")
    _need(offsets, torch.int32, (W.E + int(W.has_shared) + 1,), "offsets")
    _need(sorted_slot, torch.int32, (S,), "sorted_slot")
    _need(groups, torch.int32, (W.E + int(W.has_shared) + 1,), "groups")
    nb = workspace_bytes(MOE_OP_EXPERT_FFN, T, W.E, K, H, W.I, W.has_shared, act_mode)
    ws = _workspace(nb, dev, ws)
    st = W.struct()
    check(_lib.lib().moe_expert_ffn(ctypes.byref(st), _ptr(x), T, K, _ptr(offsets),
                                    _ptr(sorted_slot), _ptr(groups), act_mode, _ptr(y_slots),
                                    _ptr(ws), nb, _stream()))
    return (y_slots, ws) if return_ws else y_slots


def moe_expert_ffn_noalloc(W: NVFP4Weights, x: torch.Tensor, K: int, offsets: torch.Tensor,
                           sorted_slot: torch.Tensor, groups: torch.Tensor,
                           act_mode: int = MOE_ACT_BF16, y_slots: Optional[torch.Tensor] = None):
    """moe_expert_ffn with the library's fixed workspace (no caller workspace);
    pass a preallocated y_slots to allocate nothing at all."""
    _need(x, torch.bfloat16, name="x")
    T, H = x.shape
    if H != W.H:
        raise ValueError("x width does not match the weight bank")
    S = T * K + (T if W.has_shared else 0)
    y_slots = torch.empty((S, H), dtype=torch.bfloat16, device=x.device) if y_slots is None else y_slots
    _need(y_slots, torch.bfloat16, (S, H), "y_slots")
    _need(offsets, torch.int32, (W.E + int(W.has_shared) + 1,), "offsets")
    _need(sorted_slot, torch.int32, (S,), "sorted_slot")
    _need(groups, torch.int32, (W.E + int(W.has_shared) + 1,), "groups")
    st = W.struct()
    check(_lib.lib().moe_expert_ffn_noalloc(ctypes.byref(st), _ptr(x), T, K, _ptr(offsets),
                                            _ptr(sorted_slot), _ptr(groups), act_mode,
                                            _ptr(y_slots), _stream()))
    return y_slots


def moe_combine(y_slots: torch.Tensor, w: torch.Tensor, slot_pos: torch.Tensor, K: int,
                has_shared: bool, out: Optional[torch.Tensor] = None):
    _need(y_slots, torch.bfloat16, name="y_slots")
    _need(w, torch.float32, name="w")
    T = w.shape[0]
    H = y_slots.shape[1]
    _need(slot_pos, torch.int32, (T * K + (T if has_shared else 0),), "slot_pos")
    out = torch.empty((T, H), dtype=torch.bfloat16, device=y_slots.device) if out is None else out
    _need(out, torch.bfloat16, (T, H), "out")
    check(_lib.lib().moe_combine(_ptr(y_slots), _ptr(w), _ptr(slot_pos), T, K, H, int(has_shared),
                                 _ptr(out), _stream()))
    return out


def moe_combine_gated(y_slots: torch.Tensor, w: torch.Tensor, slot_pos: torch.Tensor,
                      gate: torch.Tensor, K: int, out: Optional[torch.Tensor] = None):
    """Combine with the shared expert scaled by sigmoid(gate[t])."""
    _need(y_slots, torch.bfloat16, name="y_slots")
    _need(w, torch.float32, name="w")
    T = w.shape[0]
    H = y_slots.shape[1]
    _need(slot_pos, torch.int32, (T * K + T,), "slot_pos")
    _need(gate, torch.float32, (T,), "gate")
    out = torch.empty((T, H), dtype=torch.bfloat16, device=y_slots.device) if out is None else out
    _need(out, torch.bfloat16, (T, H), "out")
    check(_lib.lib().moe_combine_gated(_ptr(y_slots), _ptr(w), _ptr(slot_pos), _ptr(gate), T, K, H,
                                       _ptr(out), _stream()))
    return out


def moe_layer(W: NVFP4Weights, x: torch.Tensor, logits: torch.Tensor, K: int,
              act_mode: int = MOE_ACT_BF16, fused: bool = False,
              gate: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
              perm=None, y_slots: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None) -> dict:
    """One layer call: route -> permute -> expert FFN -> combine, all on the GPU.
    fused=True is the C entry moe_layer (two or three kernels for decode batches; the
    permutation's outputs in `perm` = (ids, w, counts, offsets, sorted_slot,
    slot_pos, groups) when given); fused=False runs the four separate entry
    points.  Both give the same results."""
    if not fused:
        ids, w = moe_route_topk(logits, K)
        counts, offsets, sorted_slot, slot_pos, groups = moe_permute(ids, W.E, W.has_shared)
        y = moe_expert_ffn(W, x, K, offsets, sorted_slot, groups, act_mode)
        o = (moe_combine(y, w, slot_pos, K, W.has_shared) if gate is None
             else moe_combine_gated(y, w, slot_pos, gate, K))
        return dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted_slot=sorted_slot,
                    slot_pos=slot_pos, groups=groups, y_slots=y, out=o)
    _need(logits, torch.float32, name="logits")
    _need(x, torch.bfloat16, name="x")
    T, E = logits.shape
    H = x.shape[1]
    if H != W.H or E != W.E or x.shape[0] != T:
        raise ValueError("logits / x do not match the weight bank")
    hs = W.has_shared
    G = E + int(hs)
    S = T * K + (T if hs else 0)
    dev = x.device
    i32 = torch.int32
    if perm is None:
        perm = (torch.empty((T, K), dtype=i32, device=dev),
                torch.empty((T, K), dtype=torch.float32, device=dev),
                torch.empty(G, dtype=i32, device=dev), torch.empty(G + 1, dtype=i32, device=dev),
                torch.empty(S, dtype=i32, device=dev), torch.empty(S, dtype=i32, device=dev),
                torch.empty(G + 1, dtype=i32, device=dev))
    ids, w, counts, offsets, sorted_slot, slot_pos, groups = perm
    _need(ids, i32, (T, K), "ids")
    _need(w, torch.float32, (T, K), "w")
    _need(counts, i32, (G,), "counts")
    _need(offsets, i32, (G + 1,), "offsets")
    _need(sorted_slot, i32, (S,), "sorted_slot")
    _need(slot_pos, i32, (S,), "slot_pos")
    _need(groups, i32, (G + 1,), "groups")
    y_slots = torch.empty((S, H), dtype=torch.bfloat16, device=dev) if y_slots is None else y_slots
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(y_slots, torch.bfloat16, (S, H), "y_slots")
    _need(out, torch.bfloat16, (T, H), "out")
    if gate is not None:
        _need(gate, torch.float32, (T,), "gate")
    nb = workspace_bytes(MOE_OP_LAYER, T, E, K, H, W.I, hs, act_mode)
    ws = _workspace(nb, dev, ws)
    st = W.struct()
    check(_lib.lib().moe_layer(ctypes.byref(st), _ptr(logits), _ptr(x), T, K, act_mode, _ptr(gate),
                               _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets), _ptr(sorted_slot),
                               _ptr(slot_pos), _ptr(groups), _ptr(y_slots), _ptr(out), _ptr(ws), nb,
                               _stream()))
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted_slot=sorted_slot,
                slot_pos=slot_pos, groups=groups, y_slots=y_slots, out=out)


def timing_enable(on: bool = True) -> None:
    check(_lib.lib().moe_timing_enable(int(on)))


def timing_reset() -> None:
    check(_lib.lib().moe_timing_reset())


def timing_read(max_names: int = 32) -> dict:
    names = (ctypes.c_char_p * max_names)()
    launches = (ctypes.c_int * max_names)()
    ms = (ctypes.c_double * max_names)()
    dropped = ctypes.c_int(0)
    n = check(_lib.lib().moe_timing_read(names, launches, ms, max_names, ctypes.byref(dropped)))
    res = {names[i].decode(): (launches[i], ms[i]) for i in range(n)}
    if dropped.value:
        res["_dropped"] = (dropped.value, 0.0)
    return res
