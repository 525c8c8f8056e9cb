"""Element formats of NVFP4 weights, in fp64 (test infrastructure only).

* ``e2m1_decode``  -- [OCP] FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit;
  exponent field 0 is subnormal (0 or 0.5).  Pinned by the golden table of the
  16 codes and hand-worked bytes (tests/golden/e2m1_codes.txt).
* ``e4m3_decode``  -- [OCP] FP8 E4M3 "fn": bias 7, no infinities, S.1111.111 is
  NaN, largest finite 448, smallest normal 2**-6 ([attr], activations row).
  Pinned against torch.float8_e4m3fn on all 256 codes and the page facts.
* ``unpack_nibbles`` -- the resident [N, K/2] layout ([job]); low nibble holds
  the even K index (reading: the pages do not say which nibble comes first).
* ``dequant_nvfp4`` -- W = e2m1 x e4m3(block of 16 along K) x scale2 ([attr],
  weights row).  Pinned: every product equals the exact rational product.
* ``e4m3_encode_rne_sat`` -- nearest e4m3 value, ties to the even code,
  magnitudes above 448 saturate ([attr]: round-to-nearest, saturate at +-448).
  Pinned by brute-force search and by torch's e4m3 cast on in-range values.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e2m1_decode(codes) -> np.ndarray:
    """Value of 4-bit e2m1 codes (only the low 4 bits are used), as float64."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = c >> 3
    expo = (c >> 1) & 0x3
    mant = c & 0x1
    subnormal = 0.5 * mant
    normal = np.ldexp(1.0 + 0.5 * mant, expo - 1)
    mag = np.where(expo == 0, subnormal, normal).astype(np.float64)
    return np.where(sign == 1, -mag, mag)


def e4m3_decode(codes) -> np.ndarray:
    """Value of e4m3fn bytes as float64 (NaN for 0x7F and 0xFF)."""
    b = np.asarray(codes).astype(np.int64) & 0xFF
    sign = b >> 7
    expo = (b >> 3) & 0xF
    mant = b & 0x7
    subnormal = np.ldexp(mant / 8.0, -6)
    normal = np.ldexp(1.0 + mant / 8.0, expo - 7)
    mag = np.where(expo == 0, subnormal, normal).astype(np.float64)
    mag = np.where((expo == 15) & (mant == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes; element 2j is the low nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_nvfp4(codes_packed: np.ndarray, scales: np.ndarray, scale2: float = 1.0) -> np.ndarray:
    """Dequantize one [N, K/2] code matrix with its [N, K/16] e4m3 block scales.

    Every factor is exactly representable in float64 and the product of an e2m1
    value (2 significant bits), an e4m3 value (4 bits) and an fp32 (24 bits) fits
    in 53 bits, so the result is exact.
    """
    vals = e2m1_decode(unpack_nibbles(codes_packed))
    blk = np.repeat(e4m3_decode(scales), 16, axis=-1)
    assert blk.shape == vals.shape, (blk.shape, vals.shape)
    return vals * blk * float(np.float32(scale2))


def _e4m3_finite_table():
    codes = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E: all finite, >= 0
    return codes, e4m3_decode(codes)                 # values ascend with the code


def e4m3_encode_rne_sat(v) -> np.ndarray:
    """Encode values to e4m3fn bytes: nearest value, ties to even code, saturate at 448."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating e4m3 encoding here")
    codes, vals = _e4m3_finite_table()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(vals, a, side="left")        # first value >= a
    hi = np.clip(hi, 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_hi = vals[hi] - a
    d_lo = a - vals[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((codes[lo] & 1) == 0))
    pick_lo &= lo != hi
    c = np.where(pick_lo, codes[lo], codes[hi]).astype(np.int64)
    c = np.where(np.signbit(v), c | 0x80, c)
    return c.astype(np.uint8)
