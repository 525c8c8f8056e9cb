"""The bounded-error study of the MX lever (test infrastructure only): the
layer's output error, against the exact fp64 layer, when its operands are
re-encoded the way gfx950's scaled FP4/FP8 matrix instructions need them
(oracle.mx).  Run as ``python -m oracle.mx_study`` from the repository root;
tests/test_oracle_mx.py runs the same function on a small layer.

Arms (all with fp64 accumulation, so only the operand encodings differ):
  W_mxfp4[rule] : expert weights re-encoded NVFP4 -> MXFP4 (e2m1, e8m0 per 32);
                  activations exact
  x_mxfp8[rule] : weights exact; x into gate_up as MXFP8 (e4m3, e8m0 per 32)
                  -- option (b) of the prefill issue
  xh_mxfp8[rule]: also h into down as MXFP8
  full_mx[fit]  : MXFP4 weights and MXFP8 x and h (the operands of an FP4 x
                  FP8 scaled MFMA)
  fp8_row       : the FP8 arm this library runs (x per-row e4m3, h exact)
"""
from __future__ import annotations

import numpy as np

from .ffn import bf16_bits_to_f64, silu, dequant_expert
from .formats import dequant_nvfp4
from .fp8 import rowquant_dequant
from .mx import mx_quant, nvfp4_as_mxfp4
from .permute import permute
from .route import route_topk


_CACHE = {}


def _expert_weights(bank, e, wmode):
    key = (id(bank), e, wmode)
    if key in _CACHE:
        return _CACHE[key]
    if wmode is None:
        _CACHE[key] = dequant_expert(bank, e)
        return _CACHE[key]
    I = bank.I
    s2 = np.asarray(bank.scale2, dtype=np.float32)[e].astype(np.float64)
    wg = nvfp4_as_mxfp4(bank.gu_codes[e, :I], bank.gu_scales[e, :I], wmode) * s2[0]
    wu = nvfp4_as_mxfp4(bank.gu_codes[e, I:], bank.gu_scales[e, I:], wmode) * s2[1]
    wd = nvfp4_as_mxfp4(bank.dn_codes[e], bank.dn_scales[e], wmode) * s2[2]
    _CACHE[key] = (wg, wu, wd)
    return _CACHE[key]


def layer_out(x_bits, logits, bank, K, wmode=None, amode="exact", arule="ocp"):
    """Layer output [T, H] in fp64 with the operands of one arm."""
    T = x_bits.shape[0]
    x = bf16_bits_to_f64(x_bits)
    ids, w = route_topk(logits, K)
    counts, offsets, sorted_slot, slot_pos = permute(ids, bank.E, bank.has_shared)
    if amode.startswith("mxfp8"):
        xin = mx_quant(x, "e4m3", arule)
    elif amode == "fp8_row":
        xin = rowquant_dequant(x.astype(np.float32))
    else:
        xin = x
    y = np.zeros((int(offsets[-1]), bank.H))
    for e in range(len(counts)):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        sl = np.asarray(sorted_slot[a:b], dtype=np.int64)
        toks = np.where(sl < T * K, sl // K, sl - T * K)
        wg, wu, wd = _expert_weights(bank, e, wmode)
        r = xin[toks]
        h = silu(r @ wg.T) * (r @ wu.T)
        if amode == "mxfp8_xh":
            h = mx_quant(h, "e4m3", arule)
        y[a:b] = h @ wd.T
    sp = np.asarray(slot_pos, dtype=np.int64)
    out = np.zeros((T, bank.H))
    for k in range(K):
        out += w[:, k:k + 1] * y[sp[:T * K].reshape(T, K)[:, k]]
    if bank.has_shared:
        out += y[sp[T * K:]]
    return out


ARMS = {
    "W_mxfp4[ocp]": dict(wmode="ocp"),
    "W_mxfp4[fit]": dict(wmode="fit"),
    "x_mxfp8[ocp]": dict(amode="mxfp8_x", arule="ocp"),
    "x_mxfp8[fit]": dict(amode="mxfp8_x", arule="fit"),
    "xh_mxfp8[fit]": dict(amode="mxfp8_xh", arule="fit"),
    "full_mx[fit]": dict(wmode="fit", amode="mxfp8_xh", arule="fit"),
    "fp8_row": dict(amode="fp8_row"),
}


def study(wl):
    """{arm: normwise error of the layer output vs the exact layer}."""
    ref = layer_out(wl.x_bf16, wl.logits, wl.weights, wl.K)
    den = np.abs(ref).max()
    return {name: float(np.abs(layer_out(wl.x_bf16, wl.logits, wl.weights, wl.K, **kw) - ref).max() / den)
            for name, kw in ARMS.items()}


def weight_error(bank, groups=8, rule="ocp"):
    """Max and RMS of |W_mx - W| / max|W| per row, over the first groups."""
    rel_max, sq, n = 0.0, 0.0, 0
    for e in range(min(groups, bank.E)):
        w = dequant_nvfp4(bank.gu_codes[e], bank.gu_scales[e], 1.0)
        m = nvfp4_as_mxfp4(bank.gu_codes[e], bank.gu_scales[e], rule)
        d = np.abs(m - w) / np.abs(w).max(axis=1, keepdims=True)
        rel_max = max(rel_max, float(d.max()))
        sq += float((d ** 2).sum())
        n += d.size
    return rel_max, (sq / n) ** 0.5


def main():
    from workloads import make_workload, workload_for

    cases = [
        ("decode T=8 (512 experts, H=2048, I=512)", workload_for("decode", T=8)),
        ("T=16, Student-t(3) with x1000 outliers", make_workload(
            "mx", T=16, H=2048, E=512, K=10, I=512, has_shared=True, x_kind="student_t", seed=2)),
    ]
    for label, wl in cases:
        res = study(wl)
        _CACHE.clear()
        print(label)
        for k, v in res.items():
            print(f"  {k:14s} {v:.4g}")
    wl = workload_for("decode", T=1)
    for rule in ("ocp", "fit"):
        mx, rms = weight_error(wl.weights, rule=rule)
        print(f"gate_up weights, rule {rule}: max |dW|/max|W_row| {mx:.4g}, rms {rms:.4g}")


if __name__ == "__main__":
    main()
