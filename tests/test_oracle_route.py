"""Pins for the oracle router: the pages' rank rule by brute force, ties, NaN, torch, scipy."""
import math

import numpy as np
import scipy.special
import torch

import oracle
from _golden import table


def _rank_rule_ids(row, K):
    """Selection by the rank definition: rank(b) = #{j: s_j > s_b or (s_j == s_b and j < b)}."""
    s = [(-math.inf if math.isnan(v) else float(v)) for v in row]
    E = len(s)
    rank = [sum(1 for j in range(E) if s[j] > s[b] or (s[j] == s[b] and j < b)) for b in range(E)]
    by_rank = {r: b for b, r in enumerate(rank)}
    assert sorted(rank) == list(range(E))        # the rule is a total order
    return [by_rank[k] for k in range(K)]


def test_hand_worked_examples():
    for K, logits, ids, ws in table("route_examples.txt"):
        K = int(K)
        z = np.array([[float(v) for v in logits.split()]], dtype=np.float32)
        got_ids, got_w = oracle.route_topk(z, K)
        assert got_ids[0].tolist() == [int(i) for i in ids.split()]
        want = [eval(e, {"exp": math.exp}) for e in ws.split()]
        np.testing.assert_allclose(got_w[0], want, rtol=1e-15, atol=0)


def test_rank_rule_brute_force_with_ties_nan_inf():
    rng = np.random.default_rng(11)
    T, E = 60, 37
    z = (np.round(rng.normal(0, 1, (T, E)) * 4) / 4).astype(np.float32)   # many exact ties
    z[rng.random((T, E)) < 0.05] = np.nan
    z[rng.random((T, E)) < 0.03] = -np.inf
    z[5, :] = np.nan
    z[6, :] = 1.25
    for K in (1, 2, 5, 10, E):
        ids, w = oracle.route_topk(z, K)
        for t in range(T):
            assert ids[t].tolist() == _rank_rule_ids(z[t], K), (t, K)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 4e-16 * K)


def test_torch_topk_on_tie_free_rows():
    rng = np.random.default_rng(12)
    z = rng.normal(0, 1, (256, 512)).astype(np.float32)
    ids, _ = oracle.route_topk(z, 10)
    tv, ti = torch.topk(torch.from_numpy(z), 10, dim=1, largest=True, sorted=True)
    assert np.array_equal(ids, ti.numpy().astype(np.int32))


def test_weights_equal_full_softmax_restricted_and_renormalised():
    rng = np.random.default_rng(13)
    z = rng.normal(0, 3, (128, 64)).astype(np.float32)
    for K in (1, 2, 10, 64):
        ids, w = oracle.route_topk(z, K)
        p = scipy.special.softmax(z.astype(np.float64), axis=1)
        sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
        np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
        # weights are non-increasing along k (softmax is monotone in the logit)
        assert np.all(np.diff(w, axis=1) <= 0)
