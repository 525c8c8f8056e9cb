"""Token permutation grouped by expert (test infrastructure only).

Definition ([local]: the permutation is one of the dumped per-layer stages; the
layer asks for a bit-exact permutation):

* slots are (t, k) with flat index s = t*K + k;
* counts[e] = number of slots routed to expert e; with a shared expert, group E
  holds every token once (counts[E] = T);
* offsets = exclusive prefix sum of counts (length E' + 1);
* sorted_slot lists the routed slots grouped by expert, ascending slot index
  inside each group (reading: the pages fix no order inside a group; ascending
  is the stable choice and equals ascending token); the shared group follows as
  slots T*K + t for t = 0 .. T-1;
* slot_pos[s] = position of slot s in sorted_slot, for the routed slots and,
  with a shared expert, for the shared slots T*K + t as well (the inverse of
  sorted_slot over every slot; the shared group starts at offsets[E]).

Pins: pure-Python loops on random, skewed and empty-expert cases.
"""
from __future__ import annotations

import numpy as np


def permute(ids: np.ndarray, E: int, has_shared: bool):
    ids = np.asarray(ids)
    T, K = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    if has_shared:
        counts = np.concatenate([counts, [T]])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = np.argsort(flat, kind="stable")
    sorted_slot = order
    if has_shared:
        sorted_slot = np.concatenate([order, T * K + np.arange(T)])
    slot_pos = np.empty(T * K + (T if has_shared else 0), dtype=np.int64)
    slot_pos[order] = np.arange(T * K)
    if has_shared:
        slot_pos[T * K:] = offsets[E] + np.arange(T)
    return (counts.astype(np.int32), offsets, sorted_slot.astype(np.int32),
            slot_pos.astype(np.int32))
