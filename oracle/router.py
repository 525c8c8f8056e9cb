"""Router gating GEMM, routing from it, and the shared-expert gate, in fp64
(test infrastructure only).

Definition followed:

* [local] lists "the router/gating GEMM and top-k" as the first prefill op that
  changes the logits, and the per-layer dump starts with the router logits;
  [nsys] shows the router running as a w4a16 GEMM (4-bit weights, 16-bit
  activations) next to a separate router-dequant kernel ([fp4local]).
  Reading: the router matrix is NVFP4 like the experts -- e2m1 codes [R][H/2]
  (low nibble = even K index), one e4m3 scale per 16 consecutive K [R][H/16]
  and one fp32 scale2 for the whole matrix -- and the activations are the
  layer's bf16 rows.
* logits[t][e] = x_t . W_r[e] for e < E, with W_r = e2m1 x e4m3 x scale2 and x
  the exact bf16 values (every product is exact in fp64, so the sum is exact to
  fp64 rounding).
* routing is route_topk on these logits as fp32 values (the precision the
  logits are handed to the top-k in), i.e. the rule of the router stage.
* Shared-expert gate.  Reading (the pages name the shared expert but give it
  no gate; a common form is a sigmoid gate computed from the same activations):
  when the router matrix has a row E, g_t = x_t . W_r[E] and the combine scales
  the shared expert's output of token t by sigmoid(g_t); without that row the
  shared expert's weight is 1.

Pins (tests/test_oracle_router.py): pure-Python math.fsum dot products over
independently decoded weights (golden e2m1 table, torch's e4m3), scale2 powers
of two, zero codes, the gate row feeding only the gate, and routing of the
logits equals route_topk of them.
"""
from __future__ import annotations

import numpy as np

from .formats import dequant_nvfp4
from .route import route_topk


def _bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def router_logits(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                  scale2: float) -> np.ndarray:
    """x bf16 bits [T, H], codes [R, H/2], scales [R, H/16] -> fp64 [T, R]."""
    W = dequant_nvfp4(codes, scales, scale2)
    return _bf16_bits_to_f64(x_bits) @ W.T


def router_route(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, scale2: float,
                 E: int, K: int):
    """(ids, w, logits fp64 [T, E], shared gate logits fp64 [T] or None)."""
    z = router_logits(x_bits, codes, scales, scale2)
    ids, w = route_topk(z[:, :E].astype(np.float32), K)
    gate = z[:, E] if z.shape[1] > E else None
    return ids, w, z[:, :E], gate


def sigmoid(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))
    return np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
