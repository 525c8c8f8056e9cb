"""Per-token-row e4m3 activation quantisation (test infrastructure only).

Definition ([opts] option (a): row absmax taken in the gather, the row scaled
into the e4m3 range, the scale applied in the f32 epilogue; [attr]: e4m3 with
round-to-nearest and saturation at +-448).  All steps are in fp32, the precision
the quantised codes are decided in on both sides:

* amax_t = max_h |x[t, h]|  (exact in fp32);
* s_t = fp32(amax_t / 448) and inv_t = fp32(448 / amax_t), both correctly
  rounded divisions; a zero row takes s_t = inv_t = 1 (reading: the pages do not
  cover an all-zero row);
* q[t, h] = e4m3_rne_sat(fp32(x[t, h] * inv_t));
* the dequantised row is e4m3(q) * s_t.

Pins: the encoder by brute-force search and torch's cast (see formats); the
scales by exact rational arithmetic in the tests.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_decode, e4m3_encode_rne_sat


def rowquant_e4m3(x_f32: np.ndarray):
    """x float32 [T, H] -> (codes uint8 [T, H], s float32 [T])."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    amax = amax.astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    s = np.where(zero, np.float32(1.0), safe / np.float32(448.0)).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), np.float32(448.0) / safe).astype(np.float32)
    v = (x * inv[:, None]).astype(np.float32)
    return e4m3_encode_rne_sat(v), s


def rowquant_dequant(x_f32: np.ndarray) -> np.ndarray:
    """The activations the FP8 arm multiplies with: e4m3(q) * s_t, in float64."""
    q, s = rowquant_e4m3(x_f32)
    return e4m3_decode(q) * s.astype(np.float64)[:, None]
