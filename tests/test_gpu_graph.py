"""The layer call under HIP graph capture: two moe_layer calls (two logit
sets, separate output buffers) captured once and replayed three times, with
the program's own eager work and synchronisations between the replays; every
output of every replay equals the eager call's, bit for bit.  Covers the
decode layer with down + combine in one launch (T=1) and as two kernels
(T=8), the FP8 row arm with the gated combine (T=4), and a 40-token batch
through the route + permute and the fused prefill kernels."""
import pytest
import torch

from _gpu import flush, setup, x_dev
from workloads import make_workload, workload_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    return setup()


def _buffers(moe, wl, act_mode):
    T, K, E, H, I = wl.T, wl.K, wl.E, wl.H, wl.I
    hs = wl.has_shared
    G = E + int(hs)
    S = T * K + (T if hs else 0)
    i32, dev = torch.int32, "cuda"
    perm = (torch.empty((T, K), dtype=i32, device=dev),
            torch.empty((T, K), dtype=torch.float32, device=dev),
            torch.empty(G, dtype=i32, device=dev), torch.empty(G + 1, dtype=i32, device=dev),
            torch.empty(S, dtype=i32, device=dev), torch.empty(S, dtype=i32, device=dev),
            torch.empty(G + 1, dtype=i32, device=dev))
    y = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moe.workspace_bytes(4, T, E, K, H, I, hs, act_mode), dtype=torch.uint8,
                     device=dev)
    return perm, y, out, ws


def _call(moe, W, x, lg, K, act_mode, gate, bufs):
    perm, y, out, ws = bufs
    moe.moe_layer(W, x, lg, K, act_mode, fused=True, gate=gate, ws=ws, perm=perm, y_slots=y,
                  out=out)


def _outputs(bufs):
    perm, y, out, _ = bufs
    return list(perm) + [y, out]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _poison(bufs):
    for t in _outputs(bufs):
        _bits(t).fill_(0x5A5A)


CASES = {
    "decode_T1": dict(T=1, act_mode=0, gate=False),
    "decode_T8": dict(T=8, act_mode=0, gate=False),
    "decode_T4_fp8_gated": dict(T=4, act_mode=1, gate=True),
    "T40_prefill": dict(T=40, act_mode=0, gate=False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_layer_graph_replays_equal_eager(moe, case):
    c = CASES[case]
    T, act_mode = c["T"], c["act_mode"]
    flush(f"graph replay {case}")
    if T <= 8:
        wl = workload_for("decode", T=T)
        lg_b_np = workload_for("decode", T=T, seed=1, with_weights=False).logits
    else:
        shape = dict(T=T, H=1024, E=64, K=6, I=512, has_shared=True)
        wl = make_workload("graph", seed=5, **shape)
        lg_b_np = make_workload("graph", seed=6, with_weights=False, **shape).logits
    W = moe.NVFP4Weights.from_bank(wl.weights)
    x = x_dev(wl.x_bf16)
    lg_a = torch.from_numpy(wl.logits).cuda()
    lg_b = torch.from_numpy(lg_b_np).cuda()
    gate = (torch.linspace(-2.0, 2.0, T, dtype=torch.float32, device="cuda")
            if c["gate"] else None)
    bufs_a, bufs_b, bufs_o = (_buffers(moe, wl, act_mode) for _ in range(3))
    _call(moe, W, x, lg_a, wl.K, act_mode, gate, bufs_a)
    _call(moe, W, x, lg_b, wl.K, act_mode, gate, bufs_b)
    torch.cuda.synchronize()
    ref_a = [t.clone() for t in _outputs(bufs_a)]
    ref_b = [t.clone() for t in _outputs(bufs_b)]
    assert not all(torch.equal(_bits(p), _bits(q)) for p, q in zip(ref_a, ref_b))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(moe, W, x, lg_a, wl.K, act_mode, gate, bufs_a)
        _call(moe, W, x, lg_b, wl.K, act_mode, gate, bufs_b)
    torch.cuda.synchronize()
    for rep in range(3):
        _poison(bufs_a)
        _poison(bufs_b)
        torch.cuda.synchronize()
        g.replay()
        # the program's own eager work between the replays
        _call(moe, W, x, lg_b if rep % 2 else lg_a, wl.K, act_mode, gate, bufs_o)
        torch.cuda.synchronize()
        for name, got, ref in zip(("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos",
                                   "groups", "y_slots", "out"), _outputs(bufs_a), ref_a):
            assert torch.equal(_bits(got), _bits(ref)), f"replay {rep}, call a: {name}"
        for name, got, ref in zip(("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos",
                                   "groups", "y_slots", "out"), _outputs(bufs_b), ref_b):
            assert torch.equal(_bits(got), _bits(ref)), f"replay {rep}, call b: {name}"
    del g
