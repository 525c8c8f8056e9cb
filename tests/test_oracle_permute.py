"""Pins for the oracle permutation: pure-Python loops."""
import numpy as np
import pytest

import oracle


def _brute(ids, E, has_shared):
    T, K = ids.shape
    groups = [[] for _ in range(E + (1 if has_shared else 0))]
    for t in range(T):
        for k in range(K):
            groups[int(ids[t, k])].append(t * K + k)
    if has_shared:
        groups[E] = [T * K + t for t in range(T)]
    counts = [len(g) for g in groups]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    sorted_slot = [s for g in groups for s in g]
    slot_pos = [None] * (T * K + (T if has_shared else 0))
    for p, s in enumerate(sorted_slot):
        slot_pos[s] = p
    return counts, offsets, sorted_slot, slot_pos


@pytest.mark.parametrize("T,E,K,has_shared,skew", [
    (1, 8, 2, False, 0), (4, 8, 2, False, 0), (8, 512, 10, True, 0), (37, 16, 5, True, 0),
    (300, 64, 6, True, 1), (50, 512, 10, False, 1), (1, 1, 1, True, 0),
])
def test_permute_matches_loops(T, E, K, has_shared, skew):
    rng = np.random.default_rng(T * 1000 + E + K)
    z = rng.normal(0, 1, (T, E)).astype(np.float32)
    if skew:
        z += np.log(np.arange(1, E + 1) ** -2.0)[rng.permutation(E)].astype(np.float32)
    ids, _ = oracle.route_topk(z, K)
    got = oracle.permute(ids, E, has_shared)
    want = _brute(ids, E, has_shared)
    for g, w in zip(got, want):
        assert g.tolist() == list(w)
    counts = got[0]
    if skew:
        assert (counts[:E] == 0).any()     # empty experts are covered


def test_permute_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 9]]), 8, False)
