"""Seeded synthetic generators for the routed-MoE layer workloads.

Every tensor gets its own child of ``numpy.random.SeedSequence(seed)`` so that
adding a tensor never changes the others.  Conventions:

* activations ``x``: N(0,1) in fp32, then rounded to bf16 (round-to-nearest-even,
  via torch's cast); kept as the raw 16-bit patterns (``uint16``);
* router logits: N(0,1) fp32 (plus a per-expert bias for the prefill chunk,
  plus a Zipf log-prior for the long prefill);
* NVFP4 codes: uniform over all 16 e2m1 codes (so also -0), two per byte, which
  is the same as a uniform byte;
* block scales: e4m3 codes drawn uniformly from 24..72, i.e. positive values
  2**-4 .. 2**2 (codes 24 and 72 are exactly 2**-4 and 4);
* ``scale2``: one fp32 per (expert, projection in gate/up/down), 1.0.

Layout of a weight bank (E' = E + 1 when there is a shared expert, which sits
at index E):

* ``gu_codes``  uint8 [E', 2I, H/2]  rows 0..I-1 gate, I..2I-1 up; K contiguous
* ``gu_scales`` uint8 [E', 2I, H/16] one e4m3 per 16 consecutive K elements
* ``dn_codes``  uint8 [E', H, I/2]
* ``dn_scales`` uint8 [E', H, I/16]
* ``scale2``    float32 [E', 3]      (gate, up, down)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SCALE_CODE_LO = 24  # e4m3 code of 2**-4
SCALE_CODE_HI = 72  # e4m3 code of 2**2

# Stream ids for SeedSequence children; fixed so tensors never share a stream.
_S_X, _S_LOGITS, _S_BIAS, _S_PERM, _S_GU, _S_GUS, _S_DN, _S_DNS, _S_OUTL, _S_T = range(10)
_S_RC, _S_RS = 10, 11

# scale2 of a synthetic router matrix: with uniform e2m1 codes and block scales
# 2^-4 .. 4, an N(0,1) row of H = 2048 gives logits of standard deviation ~1
ROUTER_SCALE2 = 2.0 ** -8


def _rng(seed: int, stream: int) -> np.random.Generator:
    child = np.random.SeedSequence(seed).spawn(stream + 1)[stream]
    return np.random.Generator(np.random.PCG64(child))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even, torch's cast) and return the bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact: the bits move to the top half)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class WeightBank:
    E: int
    H: int
    I: int
    has_shared: bool
    gu_codes: np.ndarray
    gu_scales: np.ndarray
    dn_codes: np.ndarray
    dn_scales: np.ndarray
    scale2: np.ndarray

    @property
    def n_groups(self) -> int:
        return self.E + (1 if self.has_shared else 0)

    @property
    def bytes_per_expert(self) -> int:
        H, I = self.H, self.I
        return 2 * I * H // 2 + 2 * I * H // 16 + H * I // 2 + H * I // 16


@dataclass
class MoEWorkload:
    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    has_shared: bool
    x_bf16: np.ndarray          # uint16 [T, H]
    logits: np.ndarray          # float32 [T, E]
    weights: Optional[WeightBank] = None
    meta: dict = field(default_factory=dict)


def make_weights(E: int, H: int, I: int, has_shared: bool, seed: int = 0,
                 scale2: float = 1.0) -> WeightBank:
    assert H % 32 == 0 and I % 32 == 0
    n = E + (1 if has_shared else 0)
    gu = _rng(seed, _S_GU).integers(0, 256, size=(n, 2 * I, H // 2), dtype=np.uint8)
    gus = _rng(seed, _S_GUS).integers(SCALE_CODE_LO, SCALE_CODE_HI + 1,
                                      size=(n, 2 * I, H // 16), dtype=np.uint8)
    dn = _rng(seed, _S_DN).integers(0, 256, size=(n, H, I // 2), dtype=np.uint8)
    dns = _rng(seed, _S_DNS).integers(SCALE_CODE_LO, SCALE_CODE_HI + 1,
                                      size=(n, H, I // 16), dtype=np.uint8)
    s2 = np.full((n, 3), scale2, dtype=np.float32)
    return WeightBank(E, H, I, has_shared, gu, gus, dn, dns, s2)


@dataclass
class RouterBank:
    """NVFP4 router matrix: rows 0..E-1 route to the experts; with has_gate,
    row E is the shared-expert gate."""
    E: int
    H: int
    has_gate: bool
    codes: np.ndarray    # uint8 [R, H/2], R = E + has_gate
    scales: np.ndarray   # uint8 [R, H/16]
    scale2: float


def make_router(E: int, H: int, has_gate: bool, seed: int = 0,
                scale2: float = ROUTER_SCALE2) -> RouterBank:
    R = E + (1 if has_gate else 0)
    codes = _rng(seed, _S_RC).integers(0, 256, size=(R, H // 2), dtype=np.uint8)
    scales = _rng(seed, _S_RS).integers(SCALE_CODE_LO, SCALE_CODE_HI + 1, size=(R, H // 16),
                                        dtype=np.uint8)
    return RouterBank(E, H, has_gate, codes, scales, float(np.float32(scale2)))


def _normal_x(seed: int, T: int, H: int) -> np.ndarray:
    return _rng(seed, _S_X).standard_normal((T, H), dtype=np.float32)


def _student_t_x(seed: int, T: int, H: int, df: float = 3.0, frac: float = 1e-3,
                 mult: float = 1000.0) -> np.ndarray:
    x = _rng(seed, _S_T).standard_t(df, size=(T, H)).astype(np.float32)
    n_out = int(round(frac * T * H))
    idx = _rng(seed, _S_OUTL).choice(T * H, size=n_out, replace=False)
    flat = x.reshape(-1)
    flat[idx] *= np.float32(mult)
    return x


def zipf_log_prior(E: int, s: float, seed: int) -> np.ndarray:
    """ln p for a Zipf(s) popularity over experts, ranks assigned by a seeded permutation."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    perm = _rng(seed, _S_PERM).permutation(E)
    prior = np.empty(E, dtype=np.float64)
    prior[perm] = np.log(p)
    return prior


def make_workload(name: str, T: int, H: int, E: int, K: int, I: int, has_shared: bool,
                  seed: int = 0, x_kind: str = "normal", logit_kind: str = "normal",
                  with_weights: bool = True, bias_std: float = 0.5,
                  zipf_s: float = 1.1) -> MoEWorkload:
    if x_kind == "normal":
        xf = _normal_x(seed, T, H)
    elif x_kind == "student_t":
        xf = _student_t_x(seed, T, H)
    else:
        raise ValueError(x_kind)
    logits = _rng(seed, _S_LOGITS).standard_normal((T, E), dtype=np.float32)
    meta = {"x_kind": x_kind, "logit_kind": logit_kind, "seed": seed}
    if logit_kind == "bias":
        bias = _rng(seed, _S_BIAS).normal(0.0, bias_std, size=E).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
        meta["bias"] = bias
    elif logit_kind == "zipf":
        prior = zipf_log_prior(E, zipf_s, seed).astype(np.float32)
        logits = (logits + prior[None, :]).astype(np.float32)
        meta["prior"] = prior
    elif logit_kind != "normal":
        raise ValueError(logit_kind)
    W = make_weights(E, H, I, has_shared, seed) if with_weights else None
    return MoEWorkload(name, T, H, E, K, I, has_shared, f32_to_bf16_bits(xf), logits, W, meta)


# The five workloads of the layer: name -> keyword arguments of make_workload.
CONFIGS = {
    "tiny": dict(T=4, H=256, E=8, K=2, I=128, has_shared=False),
    "decode": dict(T=8, H=2048, E=512, K=10, I=512, has_shared=True),
    "prefill": dict(T=4096, H=2048, E=512, K=10, I=512, has_shared=True, logit_kind="bias"),
    "long_prefill": dict(T=32768, H=2048, E=512, K=10, I=512, has_shared=True,
                         logit_kind="zipf"),
    "fp8_arm": dict(T=8192, H=2048, E=512, K=10, I=512, has_shared=True,
                    x_kind="student_t"),
}
DECODE_TS = (1, 2, 4, 8)


def workload_for(name: str, seed: int = 0, T: Optional[int] = None,
                 with_weights: bool = True) -> MoEWorkload:
    kw = dict(CONFIGS[name])
    if T is not None:
        kw["T"] = T
    return make_workload(name, seed=seed, with_weights=with_weights, **kw)
