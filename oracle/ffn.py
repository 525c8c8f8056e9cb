"""Expert FFN, shared expert and combine, in fp64 (test infrastructure only).

Definitions:

* per expert e and each of its rows r (a token's activations, exact bf16 values):
  g = r . W_gate^T, u = r . W_up^T with W = dequant_nvfp4(...) x scale2 ([attr]
  weights row), rows 0..I-1 of the fused gate_up tensor being the gate and rows
  I..2I-1 the up projection (reading: the pages say "gate_up" then SiLU; gate
  first and SwiGLU h = silu(g) * u is the plain reading);
* silu(g) = g * sigmoid(g), sigmoid in the form that never overflows;
* y = h . W_down^T;
* the shared expert (index E) is one more group that holds every token with
  weight 1 (reading: the pages give it no gate);
* combine: out[t] = sum_{k<K} w[t,k] * y[slot_pos[t*K+k]] + s_t * y_shared[t]
  ([attr]: weighted sum; [tp2]: the per-slot outputs are summed in one fixed
  order -- the oracle sums in fp64, so its order does not matter here), s_t = 1,
  or sigmoid of the shared-gate logit when the router has a gate row (see
  router.py for that reading).

Options for diagnostics only: ``h_round``/``y_round`` = "bf16" round the
intermediate h or the per-slot outputs to bf16 (via torch's fp32 -> bf16 cast,
after an fp64 -> fp32 step) to mirror where the GPU stores bf16; ``act_mode`` =
"fp8_row" feeds the gate_up GEMM with the per-row e4m3-quantised activations,
"fp8_routed" / "fp8_shared" only those of the routed / the shared expert
(activation_arms).

Pins: pure-Python math.fsum loops on the tiny layer; ``bf16_bits_to_f64``
against the bf16 closed form on all 65,536 patterns and hand-worked patterns,
``_round_bf16`` against hand-worked ties, subnormals and overflow and a
brute-force nearest-value search (tests/test_oracle_bf16.py); K=1 equals the
dense FFN of the chosen expert; token permutation permutes the outputs; relabelling the
experts leaves the output unchanged; K=E equals the softmax-weighted dense
mixture; scale2 of down times 2**j scales the routed output by 2**j; all-zero
codes give zero.
"""
from __future__ import annotations

import numpy as np

from .formats import dequant_nvfp4
from .fp8 import rowquant_dequant
from .permute import permute
from .route import route_topk


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _round_bf16(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig


def dequant_expert(bank, e: int):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) of expert e in float64."""
    I = bank.I
    s2 = np.asarray(bank.scale2, dtype=np.float32)[e]
    wg = dequant_nvfp4(bank.gu_codes[e, :I], bank.gu_scales[e, :I], s2[0])
    wu = dequant_nvfp4(bank.gu_codes[e, I:], bank.gu_scales[e, I:], s2[1])
    wd = dequant_nvfp4(bank.dn_codes[e], bank.dn_scales[e], s2[2])
    return wg, wu, wd


def expert_ffn(rows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
               h_round: str = "none") -> np.ndarray:
    g = rows @ wg.T
    u = rows @ wu.T
    h = silu(g) * u
    if h_round == "bf16":
        h = _round_bf16(h)
    return h @ wd.T


def expert_outputs(xin: np.ndarray, bank, T: int, K: int, offsets, sorted_slot,
                   h_round: str = "none", groups=None, xin_shared=None) -> np.ndarray:
    """Per-slot expert outputs in sorted order: y [T*K (+T), H] float64.

    ``groups`` optionally restricts the work to some group indices (the other
    rows stay NaN), for sampled checks at full size.  ``xin_shared``, when
    given, is the activation the shared expert (group E) reads instead of xin.
    """
    n_groups = len(offsets) - 1
    y = np.full((int(offsets[-1]), bank.H), np.nan, dtype=np.float64)
    for e in (range(n_groups) if groups is None else groups):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        slots = np.asarray(sorted_slot[a:b], dtype=np.int64)
        toks = np.where(slots < T * K, slots // K, slots - T * K)
        wg, wu, wd = dequant_expert(bank, e)
        src = xin_shared if (xin_shared is not None and bank.has_shared and e == bank.E) else xin
        y[a:b] = expert_ffn(src[toks], wg, wu, wd, h_round)
    return y


def activation_arms(x: np.ndarray, act_mode: str):
    """(activations of the routed experts, of the shared expert) for an arm:
    "bf16" both exact; "fp8_row" both per-row e4m3 ([attr] option (a), the
    pages' arm E quantises routed and shared); "fp8_routed" routed e4m3 and
    the shared expert exact (the shared-expert A/B table's arm S, the shared
    expert on bf16); "fp8_shared" the mirror (routed exact, shared e4m3)."""
    if act_mode == "bf16":
        return x, x
    q = rowquant_dequant(x.astype(np.float32))
    if act_mode == "fp8_row":
        return q, q
    if act_mode == "fp8_routed":
        return q, x
    if act_mode == "fp8_shared":
        return x, q
    raise ValueError(act_mode)


def combine(y_slots: np.ndarray, w: np.ndarray, slot_pos: np.ndarray, T: int, K: int,
            has_shared: bool, shared_gate=None) -> np.ndarray:
    """out[t] = sum_k w[t,k] y[slot_pos[t*K+k]] + s_t y[slot_pos[T*K+t]], with
    s_t = sigmoid(shared_gate[t]) when gate logits are given, else 1."""
    from .router import sigmoid

    sp_all = np.asarray(slot_pos, dtype=np.int64)
    sp = sp_all[:T * K].reshape(T, K)
    out = np.zeros((T, y_slots.shape[1]), dtype=np.float64)
    for k in range(K):
        out += w[:, k:k + 1] * y_slots[sp[:, k]]
    if has_shared:
        ys = y_slots[sp_all[T * K:T * K + T]]
        if shared_gate is not None:
            ys = sigmoid(np.asarray(shared_gate, dtype=np.float64))[:, None] * ys
        out += ys
    return out


def moe_layer(x_bits: np.ndarray, logits: np.ndarray, bank, K: int, act_mode: str = "bf16",
              h_round: str = "none", y_round: str = "none") -> dict:
    """Whole layer: route -> permute -> expert FFNs (+ shared) -> combine, all fp64."""
    T = x_bits.shape[0]
    x = bf16_bits_to_f64(x_bits)
    ids, w = route_topk(logits, K)
    counts, offsets, sorted_slot, slot_pos = permute(ids, bank.E, bank.has_shared)
    xin, xin_sh = activation_arms(x, act_mode)
    y = expert_outputs(xin, bank, T, K, offsets, sorted_slot, h_round, xin_shared=xin_sh)
    yc = _round_bf16(y) if y_round == "bf16" else y
    out = combine(yc, w, slot_pos, T, K, bank.has_shared)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted_slot=sorted_slot,
                slot_pos=slot_pos, y_slots=y, out=out)
