"""OCP MX re-encoding of the layer's operands, in fp64 (test infrastructure
only): the bounded-error study of the FP4 / MX matrix-instruction lever.

The lever on the pages: "FP4 MMA over the resident layout, no dequant"
([job]) and option (b), per-16 block-scaled or MXFP8 activations ([opts]).
gfx950's scaled matrix instructions take e2m1 / e4m3 elements with one e8m0
(power-of-two) scale per 32 consecutive K elements ([OCP] MX v1.0: block size
32, one shared power-of-two scale per block).  NVFP4 weights carry one e4m3
scale per 16 ([attr], weights row), so they are not MX values in general;
this module re-encodes weights and activations as MX blocks so that the error
of the lever can be measured against the exact layer before any kernel is
written.

* e2m1_encode_rne_sat(v): nearest e2m1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6 and
  their negatives), ties to the even code, magnitudes above 6 saturate.
* mx_scale(amax, elem, rule): the block's power-of-two scale X.
  - "ocp": X = 2**(floor(log2 amax) - emax), emax the element format's largest
    exponent (2 for e2m1, whose maximum is 1.5 * 2**2; 8 for e4m3, 1.75 * 2**8):
    the OCP rule; amax / X lies in [2**emax, 2**(emax+1)), so values above the
    element maximum saturate.
  - "fit": the smallest power of two with amax / X <= the element maximum (no
    saturation, one binade coarser for the blocks the "ocp" rule would clip).
  amax = 0 gives X = 1.
* mx_quant(v, elem, rule): v [..., K] (K a multiple of 32) -> the dequantised
  MX values X * q.
* nvfp4_as_mxfp4(codes, scales, rule): the NVFP4 matrix (e2m1 x e4m3 per 16,
  scale2 left out: it stays a per-tensor factor of the f32 sums either way)
  re-encoded as MXFP4.

Pins (tests/test_oracle_mx.py): e2m1_encode_rne_sat against a brute-force
search over the decoded 16 codes, every midpoint and the saturation; the scale
rules against their closed forms; NVFP4 blocks whose two e4m3 scales are one
equal power of two survive the re-encoding exactly; every re-encoded element
lies within half a grid step (or the saturation distance) of its source.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_MAX, dequant_nvfp4, e2m1_decode, e4m3_encode_rne_sat, e4m3_decode

E2M1_MAX = 6.0
_EMAX = {"e2m1": 2, "e4m3": 8}
_MAXV = {"e2m1": E2M1_MAX, "e4m3": E4M3_MAX}
MX_BLOCK = 32


def e2m1_encode_rne_sat(v) -> np.ndarray:
    """Nearest e2m1 value of each element (ties to the even code), saturating."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    grid = e2m1_decode(np.arange(8))            # 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7)
    mid = (grid[:-1] + grid[1:]) / 2
    i = np.searchsorted(mid, a, side="left")    # the lower code of a's interval (a midpoint: the lower)
    # a midpoint between code i and i + 1 goes to the even one of the two
    at_mid = (i < 7) & (a == mid[np.minimum(i, 6)])
    i = np.where(at_mid & (i % 2 == 1), i + 1, i)
    q = grid[i]
    return np.where(v < 0, -q, q)


def mx_scale(amax, elem: str, rule: str = "ocp") -> np.ndarray:
    """Power-of-two scale X of blocks with absolute maximum amax."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    if rule == "ocp":
        e = np.floor(np.log2(safe)) - _EMAX[elem]
    elif rule == "fit":
        e = np.ceil(np.log2(safe / _MAXV[elem]))
    else:
        raise ValueError(rule)
    return np.where(amax > 0, np.ldexp(1.0, e.astype(np.int64)), 1.0)


def mx_quant(v: np.ndarray, elem: str, rule: str = "ocp") -> np.ndarray:
    """Dequantised MX values of v [..., K]: blocks of 32 along the last axis."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % MX_BLOCK == 0, "K must be a multiple of the MX block"
    b = v.reshape(v.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    X = mx_scale(np.abs(b).max(axis=-1), elem, rule)[..., None]
    if elem == "e2m1":
        q = e2m1_encode_rne_sat(b / X)
    else:
        q = e4m3_decode(e4m3_encode_rne_sat(b / X))
    return (q * X).reshape(v.shape)


def nvfp4_as_mxfp4(codes: np.ndarray, scales: np.ndarray, rule: str = "ocp") -> np.ndarray:
    """NVFP4 [N, K/2] codes with [N, K/16] e4m3 scales, re-encoded as MXFP4
    (scale2 left out), dequantised to float64 [N, K]."""
    return mx_quant(dequant_nvfp4(codes, scales, 1.0), "e2m1", rule)
