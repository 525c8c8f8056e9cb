"""GPU parity of the router (A1) and the permutation (A2): bit-exact ids and
permutation, weights within fp32 rounding of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import flush, setup
from workloads import CONFIGS, DECODE_TS, workload_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    return setup()


def _check_route(moe, logits: np.ndarray, K: int):
    ids, w = moe.moe_route_topk(torch.from_numpy(logits).cuda(), K)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route_topk(logits, K)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    wg = w.cpu().numpy().astype(np.float64)
    # fp32 exp of (z - z0) with |z - z0| ~ up to tens: relative error a few 1e-7 per
    # term; 4e-6 leaves a wide margin and still catches any wrong term
    assert np.all(np.abs(wg - w_o) <= 4e-6 * w_o + 1e-30)
    return ids


def _check_permute(moe, ids: torch.Tensor, E: int, has_shared: bool):
    got = moe.moe_permute(ids, E, has_shared)
    torch.cuda.synchronize()
    want = oracle.permute(ids.cpu().numpy(), E, has_shared)
    for g, w_, name in zip(got, want, ("counts", "offsets", "sorted_slot", "slot_pos")):
        assert np.array_equal(g.cpu().numpy(), w_), name
    active = np.nonzero(want[0])[0]
    gr = got[4].cpu().numpy()
    assert gr[0] == active.size and np.array_equal(gr[1:1 + active.size], active)
    assert np.all(gr[1 + active.size:] == -1)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "long_prefill", "fp8_arm"])
def test_route_and_permute_on_every_config(moe, name):
    Ts = DECODE_TS if name == "decode" else (None,)
    for T in Ts:
        w = workload_for(name, T=T, with_weights=False)
        flush(f"route/permute {name} T={w.T}")
        ids = _check_route(moe, w.logits, w.K)
        _check_permute(moe, ids, w.E, w.has_shared)


@pytest.mark.parametrize("seed", [0, 1])
def test_second_seed_prefill(moe, seed):
    w = workload_for("prefill", seed=seed, with_weights=False)
    ids = _check_route(moe, w.logits, w.K)
    _check_permute(moe, ids, w.E, w.has_shared)


def test_forced_ties_nan_and_infinities(moe):
    rng = np.random.default_rng(5)
    T, E = 300, 512
    z = (np.round(rng.normal(0, 1, (T, E)) * 2) / 2).astype(np.float32)   # heavy ties
    z[rng.random((T, E)) < 0.1] = np.nan
    z[rng.random((T, E)) < 0.05] = -np.inf
    z[0, :] = np.nan
    z[1, :] = -np.inf
    z[2, :] = 0.0
    z[3, :] = -0.0
    z[3, ::2] = 0.0
    z[4, 100] = np.inf
    z[4, 200] = np.inf
    for K in (1, 2, 10, 32):
        _check_route(moe, z, K)


@pytest.mark.parametrize("E,K", [(8, 8), (1, 1), (64, 1), (100, 7), (1024, 32), (37, 5)])
def test_route_shapes(moe, E, K):
    rng = np.random.default_rng(E * 100 + K)
    z = rng.normal(0, 1, (131, E)).astype(np.float32)
    ids = _check_route(moe, z, K)
    _check_permute(moe, ids, E, True)
    _check_permute(moe, ids, E, False)


@pytest.mark.parametrize("T,E,K", [(1, 512, 10), (204, 512, 10), (205, 512, 10), (5000, 64, 8),
                                   (3, 1024, 32), (777, 3, 2)])
def test_permute_with_duplicates_and_bad_ids(moe, T, E, K):
    """Ids not produced by the router: duplicates inside a token and out-of-range ids
    (slot_pos -1, counted nowhere); both paths (one workgroup / tiled) are covered."""
    rng = np.random.default_rng(T + E)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    ids[:, 0] = ids[:, -1]                              # duplicates within a token
    bad = rng.random((T, K)) < 0.02
    ids[bad] = rng.choice([-1, E, E + 5, -100], size=bad.sum())
    got = moe.moe_permute(torch.from_numpy(ids).cuda(), E, True)
    torch.cuda.synchronize()
    valid = (ids >= 0) & (ids < E)
    flat = ids.reshape(-1)
    ok = valid.reshape(-1)
    counts = np.bincount(flat[ok], minlength=E)
    order = np.nonzero(ok)[0][np.argsort(flat[ok], kind="stable")]
    offs = np.concatenate([[0], np.cumsum(np.concatenate([counts, [T]]))])
    slot_pos = np.full(T * K + T, -1)
    slot_pos[order] = np.arange(order.size)
    slot_pos[T * K:] = offs[E] + np.arange(T)       # the shared group follows the routed ones
    c, o, s, p, gr = (t.cpu().numpy() for t in got)
    active = np.nonzero(np.concatenate([counts, [T]]))[0]
    assert gr[0] == active.size and np.array_equal(gr[1:1 + active.size], active)
    assert np.all(gr[1 + active.size:] == -1)
    assert np.array_equal(c, np.concatenate([counts, [T]]))
    assert np.array_equal(o, offs)
    n_ok = order.size
    assert np.array_equal(s[:n_ok], order)
    assert np.array_equal(s[offs[E]:offs[E] + T], T * K + np.arange(T))
    assert np.array_equal(p, slot_pos)


def test_repeated_calls_are_bitwise_identical(moe):
    w = workload_for("long_prefill", with_weights=False)
    lg = torch.from_numpy(w.logits).cuda()
    a = moe.moe_route_topk(lg, w.K)
    b = moe.moe_route_topk(lg, w.K)
    pa = moe.moe_permute(a[0], w.E, True)
    pb = moe.moe_permute(b[0], w.E, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    for x, y in zip(pa, pb):
        assert torch.equal(x, y)
