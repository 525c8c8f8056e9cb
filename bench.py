#!/usr/bin/env python3
"""Benchmark of the NVFP4 routed-MoE layer on one MI355X.

A step is one whole layer call -- router top-K, permutation, expert FFN
(gate_up + SiLU + down, routed experts and the shared expert) and combine,
through moe_layer (for decode batches two or three kernels: every block of
the gate_up kernel routes and permutes the batch itself; then down and the
combine, as one launch up to 48 active groups) -- over one batch of synthetic
tokens already resident in HBM.  The
same step through the four separate entry points is timed beside it
(us_unfused).

Headline workload: the decode/verify layer at T=8 rows (H=2048, 512 experts
top-10 plus one shared expert, I=512).  Every step uses the next of NBANKS
device copies of the 907.7 MB weight bank and the next of NLOGITS router-logit
sets, so no step finds its experts in the 256 MB Infinity Cache left by the
one before.  The same loop is then run at T=1, 2, 4, on the prefill chunk
(T=4096), on the long cold prefill (T=32768, Zipf-skewed routing) and on the
FP8-arm workload (T=8192, heavy-tailed activations) in both activation arms,
as extra lines of the report, each with a CPU-oracle baseline on a bounded
sample.

The timed steps are captured once into a HIP graph and replayed, so the time
is the GPU's (the library's entry points are capturable); the eager time of
the same steps is reported beside it.  The headline follows W eager warmup
steps and one untimed replay; the extra lines, which each start after
seconds of host-side input generation, also replay their graph untimed for
~25 ms first, so that they are timed at the memory system's steady clocks.  Per-kernel durations come from HIP
events that the library records around each of its launches on the launch
stream (moe_timing_*), in an eager pass of the same steps right after.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# untimed graph replays before each timed one of the extra lines (their
# inputs are generated on the host first, seconds during which the GPU idles)
SETTLE_MS = 25.0
NBANKS = 8
NLOGITS = 16


# rocprofv3 counter summary of the expert-FFN kernels (FETCH_SIZE + WRITE_SIZE
# per dispatch, calibrated against a 1 GiB copy), with the hash of the decode
# kernel sources it was measured on.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "expert_ffn_hbm_traffic_all_workloads.md")
DECODE_SOURCES = ["bit_block_quantized_nvfp4_amd/csrc/moe_ffn_decode.hip",
                  "bit_block_quantized_nvfp4_amd/csrc/moe_ffn_common.hpp",
                  "bit_block_quantized_nvfp4_amd/csrc/moe_device.hpp",
                  "bit_block_quantized_nvfp4_amd/csrc/moe_route_permute.hpp",
                  "bit_block_quantized_nvfp4_amd/csrc/moe_topk.hpp"]


def measured_traffic():
    """HBM bytes per dec_gate_up launch (T=8) from the counter summary, or None
    if the summary is missing or the decode kernel sources changed since."""
    import hashlib
    import re

    try:
        text = open(TRAFFIC_SUMMARY).read()
        h = hashlib.sha256()
        for f in DECODE_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    m_h = re.search(r"^decode_source_sha256_16: ([0-9a-f]{16})$", text, re.M)
    if not m_b or not m_h or m_h.group(1) != h.hexdigest()[:16]:
        return None
    return int(m_b.group(1))


def _gate_up_bytes(H, I):
    return 2 * I * H // 2 + 2 * I * H // 16


def _down_bytes(H, I):
    return H * I // 2 + H * I // 16


class LayerRunner:
    """Pre-allocated buffers for one workload; run(step) enqueues one layer call."""

    def __init__(self, moe, torch, banks, wl, logits_sets, act_mode=0, fused=True):
        self.moe, self.torch = moe, torch
        self.banks, self.wl, self.act_mode, self.fused = banks, wl, act_mode, fused
        dev = "cuda"
        T, K, E, H = wl.T, wl.K, wl.E, wl.H
        hs = wl.has_shared
        S = T * K + (T if hs else 0)
        self.x = torch.from_numpy(wl.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
        self.logits = [torch.from_numpy(l).to(dev) for l in logits_sets]
        i32 = torch.int32
        self.ids = torch.empty((T, K), dtype=i32, device=dev)
        self.w = torch.empty((T, K), dtype=torch.float32, device=dev)
        G = E + int(hs)
        self.perm = (torch.empty(G, dtype=i32, device=dev), torch.empty(G + 1, dtype=i32, device=dev),
                     torch.empty(S, dtype=i32, device=dev), torch.empty(S, dtype=i32, device=dev),
                     torch.empty(G + 1, dtype=i32, device=dev))
        self.ws_p = torch.empty(max(1, moe.workspace_bytes(1, T, E, K, 0, 0, hs)), dtype=torch.uint8,
                                device=dev)
        self.ws_f = torch.empty(moe.workspace_bytes(4, T, E, K, H, wl.I, hs, act_mode),
                                dtype=torch.uint8, device=dev)   # enough for every path
        self.y = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.distinct = []

    def run(self, step):
        moe = self.moe
        W = self.banks[step % len(self.banks)]
        lg = self.logits[step % len(self.logits)]
        if self.fused:   # the one-call layer (moe_layer): the same results
            moe.moe_layer(W, self.x, lg, self.wl.K, self.act_mode, fused=True, ws=self.ws_f,
                          perm=(self.ids, self.w) + self.perm, y_slots=self.y, out=self.out)
            return
        moe.moe_route_topk(lg, self.wl.K, self.ids, self.w)
        moe.moe_permute(self.ids, self.wl.E, self.wl.has_shared, self.ws_p, self.perm)
        moe.moe_expert_ffn(W, self.x, self.wl.K, self.perm[1], self.perm[2], self.perm[4],
                           self.act_mode, self.ws_f, self.y)
        moe.moe_combine(self.y, self.w, self.perm[3], self.wl.K, self.wl.has_shared, self.out)

    def active_groups(self):
        """Distinct active groups per logits set (from the GPU's own counts)."""
        res = []
        for i in range(len(self.logits)):
            self.run(i)
            self.torch.cuda.synchronize()
            res.append(int((self.perm[0] > 0).sum().item()))
        return res


def time_steps(runner, torch, steps, warmup, graph=True, settle_ms=0.0):
    """ms per step over exactly `steps` layer calls.

    With graph=True the `steps` calls are captured once into a HIP graph
    (every library entry point is capturable: no allocation, no sync, no
    memset) and the graph is replayed: the time is the GPU's, not the Python
    launch path's.  Eager mode times the same calls launched one by one.
    settle_ms > 0 (the extra lines, which follow seconds of host-side setup):
    the graph is replayed untimed for about that long first, so the timed
    replay runs at the memory system's steady clocks (measured: the prefill
    layer read 559 us on the first replay after an idle GPU, 505-512 us once
    ~25 ms of the same traffic had run; a compute-only spin did not help).
    """
    for i in range(warmup):
        runner.run(i)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                runner.run(warmup + i)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        g.replay()                      # untimed replay
        s1.record()
        torch.cuda.synchronize()
        if settle_ms > 0:
            n = int(np.ceil(settle_ms / max(s0.elapsed_time(s1), 1e-3)))
            for _ in range(n):
                g.replay()
            torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            runner.run(warmup + i)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall


def kernel_times(runner, torch, moe_ops, steps, warmup):
    """Per-kernel durations from the HIP events the library records around each
    launch.  A short GPU spin goes first, so the whole pass is queued before
    the GPU reaches it and each event pair brackets GPU work only (not the
    host's time between recording the start event and launching the kernel)."""
    torch.cuda.synchronize()
    moe_ops.timing_reset()
    moe_ops.timing_enable(True)
    torch.cuda._sleep(int(2e7))      # ~10 ms of spinning while the host enqueues the pass
    for i in range(steps):
        runner.run(warmup + i)
    torch.cuda.synchronize()
    moe_ops.timing_enable(False)
    res = moe_ops.timing_read()
    moe_ops.timing_reset()
    return {k: {"launches": n, "avg_us": 1000.0 * ms / max(n, 1)} for k, (n, ms) in res.items()}


def cpu_baseline(wl, budget_s=12.0):
    """The fp64 oracle on the host cores, on repeated calls of the same layer."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(wl.x_bf16, wl.logits, wl.weights, wl.K)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(n * wl.T / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} fp64 oracle calls of the T={wl.T} layer (same workload, same bank), "
                      f"{dt:.1f} s, numpy BLAS threads = host cores"}


def cpu_baseline_sampled(wl, act_mode=0, budget_s=8.0):
    """The fp64 oracle on a bounded sample of a prefill-sized layer, scaled to
    the whole layer.

    The oracle's routing and permutation run on the whole config (timed); its
    expert FFN then runs on whole groups taken in a seeded random order (the
    shared group first) until the budget is spent, timing the per-group
    dequantisation and the per-row FFN apart; the combine is timed on the
    first 512 tokens.  Whole-layer time = route/permute + n_active x mean
    dequant + S x (FFN time per row) + combine x T/512.
    """
    import oracle

    cores = len(os.sched_getaffinity(0))
    T, K, E = wl.T, wl.K, wl.E
    t0 = time.perf_counter()
    ids, w = oracle.route_topk(wl.logits, K)
    counts, offsets, sorted_slot, slot_pos = oracle.permute(ids, E, wl.has_shared)
    t_rp = time.perf_counter() - t0
    x = oracle.ffn.bf16_bits_to_f64(wl.x_bf16)
    x_routed, x_shared = oracle.ffn.activation_arms(
        x, {0: "bf16", 1: "fp8_row", 2: "fp8_routed", 3: "fp8_shared"}[act_mode])
    active = [g for g in range(len(counts)) if counts[g] > 0]
    rng = np.random.default_rng(0)
    order = ([E] if wl.has_shared else []) + [int(g) for g in rng.permutation(
        [g for g in active if g != E])]
    t_dq, t_ffn, rows = [], 0.0, 0
    t_start = time.perf_counter()
    for g in order:
        a, b = int(offsets[g]), int(offsets[g + 1])
        sl = np.asarray(sorted_slot[a:b], dtype=np.int64)
        toks = np.where(sl < T * K, sl // K, sl - T * K)
        t1 = time.perf_counter()
        wg, wu, wd = oracle.ffn.dequant_expert(wl.weights, g)
        t2 = time.perf_counter()
        oracle.expert_ffn((x_shared if g == E else x_routed)[toks], wg, wu, wd)
        t3 = time.perf_counter()
        t_dq.append(t2 - t1)
        t_ffn += t3 - t2
        rows += b - a
        if len(t_dq) >= 3 and time.perf_counter() - t_start > budget_s:
            break
    n_tc = min(T, 512)
    ysub = np.zeros((n_tc * K + n_tc, wl.H))
    sp = np.concatenate([np.arange(n_tc * K), n_tc * K + np.arange(n_tc)])
    t4 = time.perf_counter()
    oracle.combine(ysub, np.asarray(w[:n_tc]), sp, n_tc, K, wl.has_shared)
    t_cb = (time.perf_counter() - t4) * T / n_tc
    S = int(offsets[-1])
    full = t_rp + len(active) * float(np.mean(t_dq)) + S * t_ffn / max(rows, 1) + t_cb
    return {"value": round(T / full, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"route+permute on all {T} tokens ({t_rp:.1f} s); {len(t_dq)} whole groups "
                      f"({rows} rows, shared group first) for dequant and FFN; combine on "
                      f"{n_tc} tokens; scaled to {len(active)} active groups and {S} rows: "
                      f"{full:.1f} s per layer call"}


COPY_BYTES = 1 << 30

WORKLOAD_TEXT = {
    "prefill": "prefill chunk: T=4096, H=2048, 512 experts top-10 + 1 shared, I=512, per-expert "
               "logit bias N(0, 0.5)",
    "long_prefill": "long cold prefill: T=32768, H=2048, 512 experts top-10 + 1 shared, I=512, "
                    "Zipf(1.1)-skewed routing",
    "fp8_arm": "FP8 arm workload: T=8192, H=2048, 512 experts top-10 + 1 shared, I=512, "
               "Student-t(3) activations with 0.1% x1000 outliers",
}


def counter_pass(moe, torch, banks, base, steps):
    """Eager layer calls for hardware-counter runs (one kernel per dispatch).

    Prints one line per phase; the counters of each kernel are read from the
    profiler's per-dispatch output.  The copy moves COPY_BYTES (read) into
    COPY_BYTES (written) with torch's elementwise copy kernel, so its
    FETCH_SIZE / WRITE_SIZE give the factor between the counters and bytes.
    """
    from workloads import workload_for

    wl = workload_for("decode", T=8, with_weights=False)
    wl.weights = base.weights
    lsets = [workload_for("decode", T=8, seed=s, with_weights=False).logits for s in range(NLOGITS)]
    r = LayerRunner(moe, torch, banks, wl, lsets)
    for i in range(steps):
        r.run(i)
    torch.cuda.synchronize()
    act = r.active_groups()
    print(f"# counter pass: decode T=8, {steps} layer calls, active groups per logits set {act}",
          file=sys.stderr, flush=True)
    for name, act_mode, calls in (("prefill", 0, 3), ("long_prefill", 0, 1), ("fp8_arm", 1, 1)):
        wl = workload_for(name, with_weights=False)
        wl.weights = base.weights
        r = LayerRunner(moe, torch, banks, wl, [wl.logits], act_mode=act_mode)
        for i in range(calls):
            r.run(i)
        torch.cuda.synchronize()
        print(f"# counter pass: {name} T={wl.T} act_mode={act_mode}, {calls} layer call(s)",
              file=sys.stderr, flush=True)
        del r
        torch.cuda.empty_cache()
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"# counter pass: 3 copies of {COPY_BYTES} bytes", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 layer calls per graph replay: the replay's own start-up (about
    # 125 us, measured) is then ~0.6 us per step instead of 2.5 us at 50
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="skip the T=1,2,4 and prefill lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--counter-pass", action="store_true",
                    help="eager launches only, for rocprofv3 --pmc: the T=8 decode layer, the T=4096, "
                         "T=32768 and FP8 T=8192 layers and a plain copy of COPY_BYTES (the counters' "
                         "scale reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the expert-parallel split is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_block_quantized_nvfp4_amd as moe
    from bit_block_quantized_nvfp4_amd import ops as moe_ops
    from workloads import CONFIGS, make_workload, workload_for

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    moe.moe_init()
    dev_name = torch.cuda.get_device_name(0)
    print(f"# device {dev_name}", file=sys.stderr, flush=True)

    base = workload_for("decode", T=8)
    bank0 = moe.NVFP4Weights.from_bank(base.weights)
    banks = [bank0]
    for _ in range(NBANKS - 1):
        banks.append(moe.NVFP4Weights(bank0.gu_codes.clone(), bank0.gu_scales.clone(),
                                      bank0.dn_codes.clone(), bank0.dn_scales.clone(),
                                      bank0.scale2.clone(), bank0.E, bank0.H, bank0.I,
                                      bank0.has_shared))
    torch.cuda.synchronize()
    H, I = base.H, base.I
    print(f"# {NBANKS} weight banks of {base.weights.bytes_per_expert * (base.E + 1) / 1e6:.1f} MB",
          file=sys.stderr, flush=True)

    if args.counter_pass:
        counter_pass(moe, torch, banks, base, args.steps)
        return

    def decode_line(T, steps, warmup, settle_ms=0.0):
        wl = workload_for("decode", T=T, with_weights=False)
        wl.weights = base.weights
        lsets = [workload_for("decode", T=T, seed=s, with_weights=False).logits for s in range(NLOGITS)]
        r = LayerRunner(moe, torch, banks, wl, lsets)
        ms, wall = time_steps(r, torch, steps, warmup, graph=True, settle_ms=settle_ms)
        ms_eager, _ = time_steps(r, torch, steps, warmup, graph=False)
        r.fused = False
        ms_unfused, _ = time_steps(r, torch, steps, warmup, graph=True, settle_ms=settle_ms)
        r.fused = True
        kt = kernel_times(r, torch, moe_ops, steps, warmup)
        act = r.active_groups()
        n_act = float(np.mean(act))
        S = T * wl.K + T
        gu_bytes = n_act * _gate_up_bytes(H, I) + T * H * 2 + S * I * 2
        dn_bytes = n_act * _down_bytes(H, I) + S * I * 2 + S * H * 2
        layer_bytes = (n_act * (_gate_up_bytes(H, I) + _down_bytes(H, I)) + 2 * T * H * 2
                       + T * wl.E * 4)
        gu = kt["dec_gate_up"]
        dn = kt["dec_down"]
        return dict(T=T, ms_per_step=ms, ms_eager=ms_eager, ms_unfused=ms_unfused, wall_s=wall,
                    tokens_per_s=T / (ms / 1e3),
                    active_groups=n_act, layer_bytes=layer_bytes,
                    layer_GBs=layer_bytes / (ms / 1e3) / 1e9, kernels=kt,
                    gate_up=dict(bytes=gu_bytes, avg_us=gu["avg_us"],
                                 GBs=gu_bytes / (gu["avg_us"] * 1e-6) / 1e9),
                    down=dict(bytes=dn_bytes, avg_us=dn["avg_us"],
                              GBs=dn_bytes / (dn["avg_us"] * 1e-6) / 1e9))

    head = decode_line(8, args.steps, args.warmup)
    print(f"# decode T=8: {head['ms_per_step'] * 1e3:.1f} us/layer, gate_up "
          f"{head['gate_up']['avg_us']:.1f} us {head['gate_up']['GBs']:.0f} GB/s, kernels {head['kernels']}",
          file=sys.stderr, flush=True)

    extra = {}
    outs = {}
    if not args.no_extra:
        for T in (1, 2, 4):
            d = decode_line(T, args.steps, args.warmup, settle_ms=SETTLE_MS)
            extra[f"decode_T{T}"] = {
                "tokens_per_s": round(d["tokens_per_s"], 1), "us_per_layer": round(d["ms_per_step"] * 1e3, 2),
                "us_per_layer_eager": round(d["ms_eager"] * 1e3, 2),
                "us_per_layer_unfused": round(d["ms_unfused"] * 1e3, 2),
                "layer_GBs": round(d["layer_GBs"], 1),
                "gate_up": {"avg_us": round(d["gate_up"]["avg_us"], 2), "GBs": round(d["gate_up"]["GBs"], 1),
                            "frac": round(d["gate_up"]["GBs"] / HBM_PEAK_GBS, 4)},
                "down": {"avg_us": round(d["down"]["avg_us"], 2), "GBs": round(d["down"]["GBs"], 1)},
                "kernels": {k: round(v["avg_us"], 2) for k, v in d["kernels"].items()}}
            print(f"# decode T={T}: {d['ms_per_step'] * 1e3:.1f} us/layer", file=sys.stderr, flush=True)
        for name, act_mode in (("prefill", 0), ("long_prefill", 0), ("fp8_arm", 1),
                               ("fp8_arm", 0), ("fp8_arm", 2)):
            wl = workload_for(name, with_weights=False)
            wl.weights = base.weights
            lsets = [workload_for(name, seed=s, with_weights=False).logits for s in range(2)]
            r = LayerRunner(moe, torch, banks, wl, lsets, act_mode=act_mode)
            ms, _ = time_steps(r, torch, args.prefill_steps, 2, graph=True, settle_ms=SETTLE_MS)
            kt = kernel_times(r, torch, moe_ops, args.prefill_steps, 2)
            S = wl.T * wl.K + wl.T
            fl_gu = 2.0 * S * H * 2 * I
            fl_dn = 2.0 * S * I * H
            suffix = {0: "_bf16" if name == "fp8_arm" else "", 1: "_fp8", 2: "_fp8_routed"}[act_mode]
            key = f"{name}_T{wl.T}" + suffix
            ent = {"workload": WORKLOAD_TEXT[name] + {0: "", 1: ", FP8 row-quantised activations",
                                                      2: ", FP8 activations for the routed experts, "
                                                         "bf16 for the shared expert"}[act_mode],
                   "tokens_per_s": round(wl.T / (ms / 1e3), 1), "us_per_layer": round(ms * 1e3, 1),
                   "layer_TFLOPs": round((fl_gu + fl_dn) / (ms / 1e3) / 1e12, 1),
                   "layer_frac": round((fl_gu + fl_dn) / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                   "kernels": {k: round(v["avg_us"], 2) for k, v in kt.items()}}
            ffn_us = sum(v["avg_us"] for k, v in kt.items() if k.startswith("grouped"))
            ent["expert_ffn"] = {"avg_us": round(ffn_us, 1),
                                 "TFLOPs": round((fl_gu + fl_dn) / (ffn_us * 1e-6) / 1e12, 1),
                                 "frac": round((fl_gu + fl_dn) / (ffn_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
            for kname, fl in (("grouped_gate_up", fl_gu), ("grouped_down", fl_dn),
                              ("grouped_ffn", fl_gu + fl_dn)):
                if kname in kt:
                    us = kt[kname]["avg_us"]
                    ent[kname] = {"avg_us": round(us, 1), "TFLOPs": round(fl / (us * 1e-6) / 1e12, 1),
                                  "frac": round(fl / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
            if name == "fp8_arm":
                r.run(0)
                torch.cuda.synchronize()
                outs[act_mode] = r.out.float().clone()
                if 0 in outs and act_mode != 0:
                    d = (outs[act_mode] - outs[0]).abs().max() / outs[0].abs().max()
                    ent["vs_bf16_path_normwise"] = round(float(d), 5)
                if act_mode == 0 and 1 in outs:
                    d = (outs[1] - outs[0]).abs().max() / outs[0].abs().max()
                    extra["fp8_arm_T8192_fp8"]["vs_bf16_path_normwise"] = round(float(d), 5)
            if not args.no_cpu:
                ent["cpu_baseline"] = cpu_baseline_sampled(wl, act_mode)   # wl.weights: the same seed-0 bank
            extra[key] = ent
            print(f"# {key}: {ms * 1e3:.1f} us/layer, kernels {kt}", file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        wl = workload_for("decode", T=8, with_weights=False)
        wl.weights = base.weights
        cpu = cpu_baseline(wl)
        print(f"# cpu baseline {cpu}", file=sys.stderr, flush=True)

    gu = head["gate_up"]
    line = {
        "metric": "MoE-layer tokens/s (decode/verify layer)",
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode/verify MoE layer: T=8 rows, H=2048, 512 routed experts top-10 "
                               "+ 1 shared, I=512, NVFP4 weights (e2m1, e4m3 per 16, fp32 scale2), "
                               "bf16 activations; 8 rotating weight banks",
                   "global_batch": 8, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "dec_gate_up", "achieved": round(gu["GBs"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gu["GBs"] / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "traffic_source": "FETCH_SIZE + WRITE_SIZE per dispatch of this kernel from "
                                       "rocprofv3 --pmc runs of bench.py --counter-pass, read from "
                                       "the profiles/ summary while the decode kernel sources hash "
                                       "to the value recorded there (else null); not measured in "
                                       "this run",
                     "layer_frac": round(head["layer_GBs"] / HBM_PEAK_GBS, 4),
                     "avg_us": round(gu["avg_us"], 2),
                     "bytes_per_launch": int(gu["bytes"])},
        "cpu_baseline": cpu,
        "layer": {"us": round(head["ms_per_step"] * 1e3, 2), "us_eager": round(head["ms_eager"] * 1e3, 2),
                  "us_unfused": round(head["ms_unfused"] * 1e3, 2),
                  "timing": "HIP graph replay of the timed steps (eager time: us_eager); the step "
                            "is moe_layer, one call (us_unfused: the four separate entry points, "
                            "same results); in moe_layer the dec_gate_up launch also routes and "
                            "permutes the batch",
                  "GBs": round(head["layer_GBs"], 1),
                  "frac": round(head["layer_GBs"] / HBM_PEAK_GBS, 4),
                  "active_groups": round(head["active_groups"], 2),
                  "kernels_avg_us": {k: round(v["avg_us"], 2) for k, v in head["kernels"].items()},
                  "down": {"avg_us": round(head["down"]["avg_us"], 2),
                           "GBs": round(head["down"]["GBs"], 1)}},
        "extra": extra,
        "device": dev_name,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
