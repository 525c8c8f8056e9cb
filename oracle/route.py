"""Router: top-K experts per token and their weights, in fp64 (test infrastructure only).

Definition followed ([A1], [topk], and the layer's "softmax top-k renormalised"):

* experts are ranked per token by their fp32 logit, larger first; equal logits
  rank the lower expert index first; a NaN logit counts as -inf;
* ids[t, k] is the expert of rank k (k = 0 .. K-1), i.e. slot k is the rank-k
  expert (reading: the pages fix the rank rule, not the slot order);
* w[t, k] = exp(z_k - z_max) / sum_j exp(z_j - z_max) over the K selected logits,
  which equals the full softmax restricted to the K experts and renormalised.
  Where z_k == z_max the term is exp(0) = 1 even for infinite logits (reading:
  the limit of the softmax; it makes an all -inf row uniform and puts all weight
  on +inf logits).

Ranking uses the logits themselves, never rounded probabilities: softmax is
monotone, so the order is the same, and fp32-rounded probabilities could create
ties that the logits do not have.

Pins (tests/test_oracle_route.py): the rank-count definition evaluated by brute
force, forced ties and NaN rows, torch.topk on tie-free rows, and scipy's full
softmax restricted and renormalised.
"""
from __future__ import annotations

import numpy as np


def route_topk(logits: np.ndarray, K: int):
    """logits float32 [T, E] -> (ids int32 [T, K], w float64 [T, K])."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = z.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    z = np.where(np.isnan(z), -np.inf, z)
    idx = np.broadcast_to(np.arange(E), z.shape)
    order = np.lexsort((idx, -z), axis=-1)          # primary: -z ascending; then index
    ids = order[:, :K].astype(np.int32)
    zs = np.take_along_axis(z, order[:, :K], axis=1)
    zmax = zs[:, :1]
    with np.errstate(invalid="ignore"):
        d = np.where(zs == zmax, 0.0, zs - zmax)
    e = np.exp(d)
    w = e / e.sum(axis=1, keepdims=True)
    return ids, w
