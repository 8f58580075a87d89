#!/usr/bin/env python3
"""GDN verify tokens/s per layer (K=16) and achieved HBM bandwidth on one MI355X.

One step is one pass of the whole hot path of one GDN layer over one verify
window, in one launch (gdn_verify_step): the rollback of the previous window
(its accept length picks the start state and the conv history), the conv step
(fused causal conv1d + SiLU, history write-back, window capture) and the gated
delta rule over K=16 tokens with every intermediate state written.  Workload:
B=1, Hk=16 key heads, Hv=48 value heads, d=128, conv width 4 over C=10240
channels, bf16 inputs and outputs, fp32 state; seeded synthetic inputs
(speculative_verify_gdn_amd.synth), accept lengths ~ U{0..16}.

Inputs are resident in HBM before timing starts.  The step cycles over R
buffer sets whose total size is at least twice the 256 MB Infinity Cache, so
the state traffic really goes to HBM; set r continues from set r-1's window as
in a serving loop.  The steps are captured in HIP graphs; after W warm-up
steps and a clock-settle phase (untimed), each of --trials timed trials
replays exactly K steps between device synchronisations, and the median trial
is the figure (min and max beside it).

Printed: one JSON line with the metric, the roofline of the step's kernel
(algorithmic bytes per launch / its median duration, timed with HIP events on
the launch stream around graph-replayed back-to-back launches of that kernel
alone; the measured device-copy and device-write rates beside the published peak), and the CPU
oracle timed on the host as a baseline (one thread and all usable cores).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials 20]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN verify tokens/s per layer (K=16) + achieved HBM GB/s vs peak"
# the sources of the step's kernel (gdn_verify_step on bf16 slabs); the committed counter profile of
# the kernel is used only while they hash to the value recorded with it
STEP_SOURCES = ("gdn_step.hip", "gdn_verify_common.h", "gdn_device.h", "gdn_conv_math.h", "gdn_timeline.h", "gdn_debug.h")
# the sources of gdn_verify with bf16 in and bf16 o (the instance the bench times)
VERIFY_SOURCES = ("gdn_verify_impl.h", "gdn_verify_bf16_bf16.hip", "gdn_verify_common.h", "gdn_device.h",
                  "gdn_conv_math.h", "gdn_timeline.h", "gdn_debug.h")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
O_DTYPE = [None]               # torch dtype of o, set in main (bf16 unless --o-f32)
MALL_BYTES = 256 * 2 ** 20     # Infinity Cache
PROFILE_DIR = os.path.join(ROOT, "profiles")


O_BYTES = 2                    # o in bf16 (fp32 is the opt-in: --o-f32)


def verify_bytes(wl, o_bytes=None) -> int:
    """Algorithmic bytes of one gdn_verify launch: every input read once,
    every output written once.

    per sequence: qkv slab K*C*ie + gates 2*K*Hv*ie + S_in Hv*dv*dk*4
                  + H (K-1)*Hv*dv*dk*4 + S_out Hv*dv*dk*4 + o K*Hv*dv*ob
    plus dt_bias and A_log (2*Hv*4) once.
    """
    o_bytes = O_BYTES if o_bytes is None else o_bytes
    ie = 2 if wl.bf16 else 4
    st = wl.Hv * wl.dv * wl.dk * 4
    per_b = wl.T * wl.C * ie + 2 * wl.T * wl.Hv * ie + st + (wl.T - 1) * st + st + wl.T * wl.Hv * wl.dv * o_bytes
    return wl.B * per_b + 2 * wl.Hv * 4


def verify_bytes_ragged(wl, lens, o_bytes=None) -> int:
    """verify_bytes for a ragged batch: sequence b reads and writes as a window of lens[b] tokens."""
    o_bytes = O_BYTES if o_bytes is None else o_bytes
    ie = 2 if wl.bf16 else 4
    st = wl.Hv * wl.dv * wl.dk * 4
    tot = 2 * wl.Hv * 4
    for L in lens:
        tot += L * wl.C * ie + 2 * L * wl.Hv * ie + st + (L - 1) * st + st + L * wl.Hv * wl.dv * o_bytes
    return tot


def verify_tree_bytes(wl, o_bytes=None) -> int:
    """Algorithmic bytes of one gdn_verify_tree launch over N = wl.T nodes: verify_bytes with every node's
    state written (N planes, no separate final state) and the parent indices read."""
    o_bytes = O_BYTES if o_bytes is None else o_bytes
    ie = 2 if wl.bf16 else 4
    st = wl.Hv * wl.dv * wl.dk * 4
    per_b = wl.T * wl.C * ie + 2 * wl.T * wl.Hv * ie + st + wl.T * st + wl.T * wl.Hv * wl.dv * o_bytes + 4 * wl.T
    return wl.B * per_b + 2 * wl.Hv * 4


def step_bytes(wl, o_bytes=None) -> int:
    """Algorithmic bytes of one gdn_verify_step launch (rollback of the previous window + conv step +
    verify with capture): per sequence the raw tokens K*C*ie and the W-1 history rows, the gates, the
    start state read once and written once as the checkpoint, H (K-1 states), S_out, o and the conv
    window (W-1+K rows); the taps C*W*4, dt_bias and A_log once; the accept lengths."""
    o_bytes = O_BYTES if o_bytes is None else o_bytes
    ie = 2 if wl.bf16 else 4
    st = wl.Hv * wl.dv * wl.dk * 4
    per_b = (wl.T * wl.C * ie + (wl.W - 1) * wl.C * ie + 2 * wl.T * wl.Hv * ie + 2 * st + (wl.T - 1) * st + st
             + wl.T * wl.Hv * wl.dv * o_bytes + (wl.W - 1 + wl.T) * wl.C * ie + 4)
    return wl.B * per_b + wl.C * wl.W * 4 + 2 * wl.Hv * 4


def conv_bytes(wl) -> int:
    """x read, hist read + written, y written, window written, taps read."""
    ie = 2 if wl.bf16 else 4
    return wl.B * (wl.T * wl.C * ie * 2 + (wl.W - 1) * wl.C * ie * 2 + (wl.W - 1 + wl.T) * wl.C * ie) \
        + wl.C * wl.W * 4


def rollback_bytes(wl, accept) -> int:
    """State copy (read + write) and conv-history copy for every sequence that rolls back."""
    ie = 2 if wl.bf16 else 4
    st = wl.Hv * wl.dv * wl.dk * 4
    n = sum(1 for a in accept if a < wl.T)
    return n * (2 * st + 2 * (wl.W - 1) * wl.C * ie) + 4 * wl.B


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "speculative_verify_gdn_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, "%s.%s.pmc.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_info():
    """The host's logical CPU count, the CPUs this process may run on, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def cpu_baseline(wl, budget_s: float):
    """The oracle (C: float conv, double GDN with capture, rollback) on the same workload, on the
    host: one thread, then one thread per group of key heads (up to the usable CPUs, at most one
    per key head), each calling the unchanged oracle functions on its own heads and their conv
    channels (key heads and their value heads are independent; the ctypes calls release the
    GIL).  Each leg: one warm-up step, then 5 runs of about budget/10 seconds each; the median
    run is reported with the minimum and maximum."""
    import concurrent.futures
    import statistics

    import numpy as np

    import oracle
    from speculative_verify_gdn_amd import synth

    inp = synth.make_inputs(wl, seed=0)
    x = inp["x"].float().numpy()
    w = inp["w"].numpy()
    hist = inp["hist"].float().numpy()
    f = lambda k: inp[k].double().numpy()
    br, al, dt, alog, S_in = f("beta_raw"), f("alpha"), f("dt_bias"), f("A_log"), f("S_in")
    acc = inp["accept"].numpy()
    o = oracle.default()
    grp = wl.Hv // wl.Hk

    def part(k0, k1):
        # the sub-problem of key heads k0..k1-1: their q and k channels, their value heads' v channels
        h0, h1 = k0 * grp, k1 * grp
        qk = wl.Hk * wl.dk
        idx = np.concatenate([np.arange(k0 * wl.dk, k1 * wl.dk), qk + np.arange(k0 * wl.dk, k1 * wl.dk),
                              2 * qk + np.arange(h0 * wl.dv, h1 * wl.dv)])
        c = np.ascontiguousarray
        return dict(x=c(x[..., idx]), w=c(w[idx]), hist=c(hist[..., idx]), br=c(br[..., h0:h1]),
                    al=c(al[..., h0:h1]), dt=c(dt[h0:h1]), alog=c(alog[h0:h1]), S_in=c(S_in[:, h0:h1]),
                    Hk=k1 - k0)

    def step(pt):
        y, hist_out, win = o.conv_step_f32(pt["x"], pt["w"], pt["hist"], round_bf16=wl.bf16)
        S_out, H, _ = o.gdn_recurrent_f64(y.astype(np.float64), pt["br"], pt["al"], pt["dt"], pt["alog"],
                                          pt["S_in"], pt["Hk"])
        o.rollback(acc, wl.T, pt["S_in"], H, S_out, win=win, hist=hist_out)
        return S_out

    def leg(parts):
        with concurrent.futures.ThreadPoolExecutor(len(parts)) as ex:
            def one():
                list(ex.map(step, parts))
            t0 = time.perf_counter()
            one()                                    # warm-up
            t_step = time.perf_counter() - t0
            n = max(1, math.ceil(budget_s / 10 / max(t_step, 1e-6)))
            runs = []
            for _ in range(5):
                t0 = time.perf_counter()
                for _ in range(n):
                    one()
                runs.append(n * wl.B * wl.T / (time.perf_counter() - t0))
        return {"value": round(statistics.median(runs), 1), "min": round(min(runs), 1), "max": round(max(runs), 1),
                "steps_per_run": n, "threads": len(parts)}

    info = host_info()
    whole = part(0, wl.Hk)
    single = leg([whole])
    nt = max(1, min(info["usable_cpus"] or 1, wl.Hk))
    bounds = [round(i * wl.Hk / nt) for i in range(nt + 1)]
    parts = [part(bounds[i], bounds[i + 1]) for i in range(nt)]
    # the key-head groups together give the whole problem's states, bit for bit
    assert np.array_equal(np.concatenate([step(pt) for pt in parts], axis=1), step(whole))
    multi = leg(parts)
    return {"value": multi["value"], "unit": "tokens/s", "cores": multi["threads"], "kind": "oracle",
            "sample": "the %s workload (float conv + double GDN with capture + rollback): one warm-up step, then "
                      "5 runs of %d full steps on %d threads (one key-head group each); median run" %
                      (wl.name, multi["steps_per_run"], multi["threads"]),
            "min": multi["min"], "max": multi["max"], "single_thread": single, **info}


def other_workloads(torch, gdn, synth, dev, only=("decode", "batched", "tree", "prefill")):
    """Kernel time of gdn_verify on the decode (K=1) and batched (B=32, K=8)
    workloads, and of gdn_prefill_chunked on the prefill workload (B=4 x
    T=4096, chunk 64): graph-replayed back-to-back launches over enough buffer
    sets to exceed the Infinity Cache, HIP events on the launch stream."""
    res = {}

    def timed(fn, sets, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for d in sets:
                fn(d)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(sets))

    for name in [n for n in ("decode", "batched") if n in only]:
        wl = synth.WORKLOADS[name]
        per = wl.B * wl.Hv * wl.dv * wl.dk * 4 * (wl.T + 1)
        R = max(2, math.ceil(2 * MALL_BYTES / per))
        sets = []
        for r in range(R):
            inp = synth.make_inputs(wl, seed=r)
            d = {k: v.to(dev) for k, v in inp.items()}
            d["qkv"] = synth.make_qkv(wl, seed=r).to(dev)
            d["S_out"] = torch.empty_like(d["S_in"])
            d["H"] = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device=dev) if wl.T > 1 else None
            d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=O_DTYPE[0])
            sets.append(d)

        def ver(d, wl=wl):
            gdn.verify(d["qkv"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"],
                       d["H"], d["o"], wl.Hk)
        us = timed(ver, sets, max(1, 200 // R))
        b = verify_bytes(wl)
        res[name] = {"verify_us": round(us, 3), "bytes_per_launch": b, "GBs": round(b / (us * 1e-6) / 1e9, 1),
                     "tokens_per_s": round(wl.B * wl.T / (us * 1e-6), 1)}
        del sets
    if "batched" in only:
        # the same batch with per-sequence verify lengths drawn U{1..8} (one launch, lens on the device)
        wl = synth.WORKLOADS["batched"]
        g = torch.Generator().manual_seed(5)
        lens = torch.randint(1, wl.T + 1, (wl.B,), generator=g, dtype=torch.int32)
        per = sum((int(L) + 1) for L in lens) * wl.Hv * wl.dv * wl.dk * 4
        R = max(2, math.ceil(2 * MALL_BYTES / per))
        sets = []
        for r in range(R):
            inp = synth.make_inputs(wl, seed=r)
            d = {k: v.to(dev) for k, v in inp.items()}
            d["qkv"] = synth.make_qkv(wl, seed=r).to(dev)
            d["S_out"] = torch.empty_like(d["S_in"])
            d["H"] = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device=dev)
            d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=O_DTYPE[0])
            d["lens"] = lens.to(dev)
            sets.append(d)

        def ver_r(d, wl=wl):
            gdn.verify(d["qkv"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"],
                       d["H"], d["o"], wl.Hk, lens=d["lens"])
        us = timed(ver_r, sets, max(1, 200 // R))
        b = verify_bytes_ragged(wl, [int(L) for L in lens])
        res["batched_ragged"] = {"verify_us": round(us, 3), "lens_total": int(lens.sum()), "bytes_per_launch": b,
                                 "GBs": round(b / (us * 1e-6) / 1e9, 1),
                                 "tokens_per_s": round(int(lens.sum()) / (us * 1e-6), 1)}
        del sets
    for name in [n for n in ("decode", "batched") if n in only]:
        # the whole step in one launch (gdn_verify_step) against the separate launches, sets chained as in
        # a serving loop (set r continues from set r-1's window)
        wl = synth.WORKLOADS[name]
        per = wl.B * wl.Hv * wl.dv * wl.dk * 4 * (wl.T + 2)
        R = max(2, math.ceil(2 * MALL_BYTES / per))
        sets = []
        for r in range(R):
            inp = synth.make_inputs(wl, seed=r)
            d = {k: v.to(dev) for k, v in inp.items()}
            d["S_ckpt"] = torch.empty_like(d["S_in"])
            d["S_out"] = torch.empty_like(d["S_in"])
            d["H"] = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device=dev) if wl.T > 1 else None
            d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=O_DTYPE[0])
            d["y"] = torch.empty_like(d["x"])
            d["win"] = torch.empty(wl.B, wl.W - 1 + wl.T, wl.C, device=dev, dtype=d["x"].dtype)
            d["win_prev"] = torch.empty_like(d["win"])
            sets.append(d)
        for d in sets:
            gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_out"], d["H"],
                            d["o"], wl.Hk, S_in=d["S_in"], hist=d["hist"], S_ckpt=d["S_ckpt"], win=d["win"])
            gdn.conv_step(d["x"], d["w"], d["hist"].clone(), d["y"], d["win_prev"])
        idx = {id(d): r for r, d in enumerate(sets)}

        def fused(d, wl=wl):
            pv = sets[idx[id(d)] - 1]
            gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_out"], d["H"],
                            d["o"], wl.Hk, prev=(pv["accept"], pv["S_ckpt"], pv["H"], pv["S_out"], pv["win"]),
                            S_ckpt=d["S_ckpt"], win=d["win"])

        def two(d, wl=wl):
            gdn.rollback_conv_step(d["accept"], wl.T, d["S_in"], d["H"], d["S_out"], d["win_prev"], d["x"], d["w"],
                                   d["hist"], d["y"], d["win"])
            gdn.verify(d["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"], d["H"],
                       d["o"], wl.Hk)
        reps = max(1, 200 // R)
        t_f, t_2 = timed(fused, sets, reps), timed(two, sets, reps)
        res[name + "_step"] = {"verify_step_us": round(t_f, 3), "two_launch_step_us": round(t_2, 3),
                               "tokens_per_s": round(wl.B * wl.T / (t_f * 1e-6), 1),
                               "step_bytes_per_launch": step_bytes(wl),
                               "GBs": round(step_bytes(wl) / (t_f * 1e-6) / 1e9, 1)}
        del sets
    if "batched" in only:
        # rollback by capture (verify writes every H_t, rollback copies H_{a-1}) against checkpoint + replay
        # (verify writes the final state only, replay re-runs the accepted prefix from S_in), state only,
        # accept lengths drawn U{0..K} (seed 6)
        wl = synth.WORKLOADS["batched"]
        g = torch.Generator().manual_seed(6)
        acc = torch.randint(0, wl.T + 1, (wl.B,), generator=g, dtype=torch.int32)
        per = wl.B * wl.Hv * wl.dv * wl.dk * 4 * (wl.T + 1)
        R = max(2, math.ceil(2 * MALL_BYTES / per))
        sets = []
        for r in range(R):
            inp = synth.make_inputs(wl, seed=r)
            d = {k: v.to(dev) for k, v in inp.items()}
            d["qkv"] = synth.make_qkv(wl, seed=r).to(dev)
            d["S_out"] = torch.empty_like(d["S_in"])
            d["H"] = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device=dev)
            d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=O_DTYPE[0])
            d["acc"] = acc.to(dev)
            sets.append(d)

        def cap(d, wl=wl):
            gdn.verify(d["qkv"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"],
                       d["H"], d["o"], wl.Hk)
            gdn.rollback(d["acc"], wl.T, d["S_in"], d["H"], d["S_out"])

        def rep(d, wl=wl):
            gdn.verify(d["qkv"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"],
                       None, d["o"], wl.Hk)
            gdn.replay(d["acc"], d["qkv"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"],
                       d["S_out"], wl.Hk)
        reps = max(1, 200 // R)
        res["batched_rollback"] = {"accept_total": int(acc.sum()), "capture_step_us": round(timed(cap, sets, reps), 3),
                                   "replay_step_us": round(timed(rep, sets, reps), 3),
                                   "steps": "verify(H) + rollback vs verify(no H) + replay, state only"}
        del sets
    if "tree" in only:
        # tree verify on the verify16 shape: N = 16 and 32 nodes of a random draft tree (parent among the 4
        # previous nodes) and of a breadth-first binary tree; the conv of every node, the verify, and the
        # rollback to a drawn node
        for N, shape in ((16, "random"), (32, "random"), (16, "binary"), (32, "binary")):
            wl = synth.small("verify16", T=N)
            per = wl.B * wl.Hv * wl.dv * wl.dk * 4 * (N + 1)
            R = max(2, math.ceil(2 * MALL_BYTES / per))
            sets = []
            for r in range(R):
                inp = synth.make_inputs(wl, seed=r)
                d = {k: v.to(dev) for k, v in inp.items()}
                d["parent"] = synth.make_tree(wl.B, N, seed=r, shape=shape).to(dev)
                d["node"] = synth.make_tree_accept(wl.B, N, seed=r).to(dev)
                d["y"] = torch.empty_like(d["x"])
                d["S_out"] = torch.empty_like(d["S_in"])
                d["H"] = torch.empty(wl.B, N, wl.Hv, wl.dv, wl.dk, device=dev)
                d["o"] = torch.empty(wl.B, N, wl.Hv, wl.dv, device=dev)
                d["S_ckpt"] = torch.empty_like(d["S_in"])
                d["hist_out"] = torch.empty_like(d["hist"])
                sets.append(d)
            tidx = {id(d): r for r, d in enumerate(sets)}

            def tfused(d, wl=wl, first=False):
                # gdn_verify_tree_step: set r continues from set r-1's tree (its accepted node, states, tokens)
                pv = sets[tidx[id(d)] - 1]
                if first:
                    gdn.verify_tree_step(d["x"], d["w"], d["parent"], d["beta_raw"], d["alpha"], d["dt_bias"],
                                         d["A_log"], d["H"], d["o"], d["y"], wl.Hk, d["S_in"], d["hist"],
                                         S_ckpt=d["S_ckpt"], hist_out=d["hist_out"])
                else:
                    gdn.verify_tree_step(d["x"], d["w"], d["parent"], d["beta_raw"], d["alpha"], d["dt_bias"],
                                         d["A_log"], d["H"], d["o"], d["y"], wl.Hk, pv["S_ckpt"], pv["hist_out"],
                                         prev=(pv["node"], pv["parent"], pv["H"], pv["x"]), S_ckpt=d["S_ckpt"],
                                         hist_out=d["hist_out"])

            def tconv(d):
                gdn.conv_tree(d["x"], d["w"], d["hist"], d["parent"], d["y"])

            def tver(d, wl=wl):
                gdn.verify_tree(d["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["parent"], d["S_in"],
                                d["H"], d["o"], wl.Hk)

            def troll(d):
                gdn.rollback_tree(d["node"], d["parent"], d["S_in"], d["H"], d["S_out"], d["x"], d["hist"])

            def tstep(d):
                tconv(d)
                tver(d)
                troll(d)
            for fn in sets:
                tconv(fn)
                tfused(fn, first=True)
            reps = max(1, 200 // R)
            t_v = timed(tver, sets, reps)
            t_s = timed(tstep, sets, reps)
            t_f = timed(tfused, sets, reps)
            b = verify_tree_bytes(wl)
            res["tree%d%s" % (N, "" if shape == "random" else "_" + shape)] = {
                                 "verify_tree_us": round(t_v, 3), "bytes_per_launch": b,
                                 "GBs": round(b / (t_v * 1e-6) / 1e9, 1),
                                 "conv_tree_us": round(timed(tconv, sets, reps), 3),
                                 "rollback_tree_us": round(timed(troll, sets, reps), 3),
                                 "step_us": round(t_s, 3), "nodes_per_s": round(N / (t_s * 1e-6), 1),
                                 "fused_step_us": round(t_f, 3),
                                 "tree": {"random": "random, parent among the 4 previous nodes",
                                          "binary": "complete binary, breadth-first numbering"}[shape]}
            del sets
    if "prefill" not in only:
        return res
    wl = synth.WORKLOADS["prefill"]
    inp = synth.make_inputs(wl, seed=0)
    d = {k: v.to(dev) for k, v in inp.items()}
    d["qkv"] = synth.make_qkv(wl, seed=0).to(dev)
    d["S_out"] = torch.empty_like(d["S_in"])
    d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=torch.bfloat16)

    def pre(d):
        gdn.prefill_chunked(d["qkv"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"],
                            d["o"], wl.Hk, chunk=wl.chunk)
    us = timed(pre, [d], 5)
    ie = 2
    byts = wl.B * wl.T * (wl.C * ie + 2 * wl.Hv * ie + wl.Hv * wl.dv * 2) + 2 * wl.B * wl.Hv * wl.dv * wl.dk * 4
    # multiply-adds of the chunkwise form per (sequence, head, chunk of L tokens): S K^T, S Q^T and
    # the state update (3 dv dk L), K K^T and Q K^T lower halves (L^2 dk), the triangular solve and
    # M U lower halves (L^2 dv); the ragged last chunk counted whole
    L = wl.chunk
    chunks = -(-wl.T // L)
    macs = wl.B * wl.Hv * chunks * (3 * wl.dv * wl.dk * L + L * L * (wl.dk + wl.dv))
    res["prefill"] = {"us": round(us, 1), "tokens_per_s": round(wl.B * wl.T / (us * 1e-6), 1),
                      "bytes_per_launch": byts, "GBs": round(byts / (us * 1e-6) / 1e9, 1),
                      "chunkwise_flop_per_launch": 2 * macs,
                      "chunkwise_TFLOPs": round(2 * macs / (us * 1e-6) / 1e12, 2)}
    return res


def copy_peak(torch, dev, mib=512, trials=5):
    """A plain device copy of mib MiB (torch's copy kernel), replayed from a HIP graph: bytes read plus
    bytes written per second, median of the trials; the practical HBM ceiling next to the published
    peak."""
    import statistics
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(4):
            dst.copy_(src)
    g.replay()
    torch.cuda.synchronize()
    runs = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        runs.append(2 * n * 4 * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return {"GBs": round(statistics.median(runs), 1), "min": round(min(runs), 1), "max": round(max(runs), 1),
            "bytes_per_copy": 2 * n * 4, "copy": "%d MiB device to device (torch copy kernel), read + write" % mib}


def write_peak(torch, dev, mib=1024, trials=5, step_bytes_=0, sets=10):
    """Plain device writes (torch's fill kernel, no reads), replayed from HIP graphs, median of the trials:
    one buffer of mib MiB (the sustained write rate, 4x the Infinity Cache), and -- when step_bytes_ is given --
    `sets` buffers of that size filled back to back, one fill per launch (the step's store volume in the bench's
    rotation of buffer sets: the time a kernel that only wrote those bytes would take per launch)."""
    import statistics

    def rate(bufs, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                for b in bufs:
                    b.fill_(1.0)
        g.replay()
        torch.cuda.synchronize()
        runs = []
        for _ in range(trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e3 / (reps * len(bufs)))   # us per fill
        return statistics.median(runs), min(runs), max(runs)

    n = mib * 2 ** 20 // 4
    big = torch.empty(n, device=dev)
    us, lo, hi = rate([big], 4)
    del big
    out = {"GBs": round(n * 4 / (us * 1e-6) / 1e9, 1), "min": round(n * 4 / (hi * 1e-6) / 1e9, 1),
           "max": round(n * 4 / (lo * 1e-6) / 1e9, 1), "bytes_per_fill": n * 4,
           "write": "%d MiB device fill (torch fill kernel), writes only" % mib}
    if step_bytes_:
        m = step_bytes_ // 4
        bufs = [torch.empty(m, device=dev) for _ in range(sets)]
        us, lo, hi = rate(bufs, 2)
        del bufs
        out["step_sized"] = {"us_per_fill": round(us, 3), "GBs": round(m * 4 / (us * 1e-6) / 1e9, 1),
                             "bytes_per_fill": m * 4, "sets": sets,
                             "fill": "%d buffers of the step's state bytes, one fill per launch, back to back" % sets}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="verify16")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets cycled (0: enough to exceed 2x the MALL)")
    ap.add_argument("--eager", action="store_true", help="launch every step from Python instead of HIP graphs")
    ap.add_argument("--two-kernel", action="store_true",
                    help="step as rollback_conv_step -> verify (two launches) instead of the fused gdn_verify_step")
    ap.add_argument("--three-kernel", action="store_true",
                    help="step as conv_step -> verify -> rollback (three launches) instead of "
                         "rollback_conv_step -> verify")
    ap.add_argument("--trials", type=int, default=20,
                    help="timed trials of K steps each; the median trial is reported, with min and max")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="after the W warm-up steps, replay the step for at least this long (untimed) so the "
                         "GPU's clocks have settled before the timed trials")
    ap.add_argument("--o-f32", action="store_true", help="fp32 outputs o (default bf16)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the decode / batched / prefill kernel timings in the detail object")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time gdn_prefill_chunked on the prefill workload (B=4 x T=4096) and print its figures")
    ap.add_argument("--only", default="", metavar="NAMES",
                    help="comma-separated subset of decode,batched,tree,prefill: time only those workloads, print "
                         "their figures and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (HBM counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the verify step shards "
              "by key-head group or by sequence with no exchange between GPUs). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import statistics

    import torch

    from speculative_verify_gdn_amd import gdn, synth

    global O_BYTES
    O_DTYPE[0] = torch.float32 if args.o_f32 else torch.bfloat16
    O_BYTES = 4 if args.o_f32 else 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.copy_probe:
        # a copy of known size: each launch reads and writes exactly n bytes
        n = args.copy_probe * 2 ** 20
        src = torch.ones(n // 4, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return

    gdn.load()
    if args.prefill_only:
        print(json.dumps({"prefill": other_workloads(torch, gdn, synth, dev, only=("prefill",))["prefill"]}))
        return
    if args.only:
        print(json.dumps(other_workloads(torch, gdn, synth, dev, only=tuple(args.only.split(",")))))
        return

    wl = synth.WORKLOADS[args.workload]
    assert wl.chunk == 0, "the bench step is the verify path"

    # ---------------------------------------------------------------- buffers
    def make_set(seed):
        inp = synth.make_inputs(wl, seed=seed)
        d = {k: v.to(dev) for k, v in inp.items()}
        d["y"] = torch.empty_like(d["x"])
        d["win"] = torch.empty(wl.B, wl.W - 1 + wl.T, wl.C, dtype=d["x"].dtype, device=dev)
        d["win_prev"] = torch.empty_like(d["win"])   # the previous step's window (fused step)
        d["S_out"] = torch.empty_like(d["S_in"])
        d["H"] = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device=dev) if wl.T > 1 else None
        d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=O_DTYPE[0])
        d["S_ckpt"] = torch.empty_like(d["S_in"])     # the fused step's checkpoint (start state)
        return d

    probe = make_set(0)
    set_bytes = sum(t.numel() * t.element_size() for t in probe.values() if t is not None)
    R = args.sets or max(2, math.ceil(2 * MALL_BYTES / set_bytes))
    sets = [probe] + [make_set(r) for r in range(1, R)]
    accepts = [int(s["accept"][0]) for s in sets]

    def conv(d):
        gdn.conv_step(d["x"], d["w"], d["hist"], d["y"], d["win"])

    def verify(d):
        gdn.verify(d["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"], d["H"],
                   d["o"], wl.Hk)

    def rollback(d):
        gdn.rollback(d["accept"], wl.T, d["S_in"], d["H"], d["S_out"], d["hist"], d["win"])

    def rollback_conv(d):
        # the rollback of this set's previous window, then this step's conv, in one launch
        gdn.rollback_conv_step(d["accept"], wl.T, d["S_in"], d["H"], d["S_out"], d["win_prev"], d["x"], d["w"],
                               d["hist"], d["y"], d["win"])

    def set_index(d):
        return next(r for r, s2 in enumerate(sets) if s2 is d)

    def fused_first(d):
        # a first window (from S_in and hist): fills the checkpoint, capture and window of a set
        gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_out"], d["H"],
                        d["o"], wl.Hk, S_in=d["S_in"], hist=d["hist"], S_ckpt=d["S_ckpt"], win=d["win"])

    def fused(d):
        # one whole step in one launch, chained as in a serving loop: set r continues from set r-1's
        # window (its accept length picks the start state and the conv history) and writes its own
        pv = sets[set_index(d) - 1]
        gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_out"], d["H"],
                        d["o"], wl.Hk, prev=(pv["accept"], pv["S_ckpt"], pv["H"], pv["S_out"], pv["win"]),
                        S_ckpt=d["S_ckpt"], win=d["win"])

    mode = "three" if args.three_kernel else ("two" if args.two_kernel else "fused")
    if mode == "three":
        def step(d):
            conv(d)
            verify(d)
            rollback(d)
    elif mode == "two":
        def step(d):
            rollback_conv(d)
            verify(d)
    else:
        step = fused

    # a valid previous window for rollback_conv_step (one conv step into win_prev), and for the fused
    # step a first window of every set
    for d in sets:
        gdn.conv_step(d["x"], d["w"], d["hist"], d["y"], d["win_prev"])
        fused_first(d)

    # ---------------------------------------------------------------- warmup
    for s in range(args.warmup):
        step(sets[s % R])
    torch.cuda.synchronize()

    graphs = None
    per_graph = 1
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for d in sets:
                step(d)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        # steps back to back as in a serving loop: one graph holds one step on
        # each of the R buffer sets (when K is a multiple of R), else one graph
        # per set
        per_graph = R if args.steps % R == 0 else 1
        graphs = []
        for i in range(0, R, per_graph):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for d in sets[i:i + per_graph]:
                    step(d)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- clock settle (untimed)
    settle_t0 = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - settle_t0) * 1e3 < args.settle_ms:
        if graphs is not None:
            for g in graphs:
                g.replay()
            settle_steps += per_graph * len(graphs)
        else:
            for d in sets:
                step(d)
            settle_steps += R
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    # trials of exactly K steps each, bracketed by device synchronisations; the median trial is
    # the figure
    K = args.steps
    trial_ms = []
    w0 = time.perf_counter()
    for _ in range(max(1, args.trials)):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        if graphs is not None:
            for s_ in range(K // per_graph):
                graphs[s_ % len(graphs)].replay()
        else:
            for s_ in range(K):
                step(sets[s_ % R])
        ev1.record()
        torch.cuda.synchronize()
        trial_ms.append(ev0.elapsed_time(ev1) / K)
    wall_ms = (time.perf_counter() - w0) * 1e3
    ms_per_step = statistics.median(trial_ms)
    tokens = wl.B * wl.T
    value = tokens / (ms_per_step * 1e-3)

    # ---------------------------------------------------------------- per-kernel durations
    # each kernel alone, back to back over the R buffer sets: one HIP graph of
    # R launches per kernel, replayed; HIP events on the launch stream bracket
    # the replays, so the figure is the kernel's duration plus the GPU's own
    # gap between consecutive kernels (no host launch cost)
    def kernel_us(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for d in sets:
                fn(d)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, min(K, 400) // R)
        runs = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e3 / (reps * R))
        return statistics.median(runs)

    if args.eager:
        def kernel_us(fn):  # noqa: F811  (events around each eager launch)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(min(K, 200))]
            torch.cuda.synchronize()
            for s, (e0, e1) in enumerate(evs):
                e0.record()
                fn(sets[s % R])
                e1.record()
            torch.cuda.synchronize()
            return sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs) * 1e3

    t_fused = kernel_us(fused)

    # resident: the same chained step on two buffer sets only (each continues from the other), whose
    # working set fits the 256 MB Infinity Cache -- reported beside the HBM-bound figure, labelled
    def resident_us():
        def fused_from(d, pv):
            gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_out"], d["H"],
                            d["o"], wl.Hk, prev=(pv["accept"], pv["S_ckpt"], pv["H"], pv["S_out"], pv["win"]),
                            S_ckpt=d["S_ckpt"], win=d["win"])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(5):
                fused_from(sets[0], sets[1])
                fused_from(sets[1], sets[0])
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, min(K, 400) // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * 10)

    t_resident = resident_us() if (mode == "fused" and R >= 2 and not args.eager) else None
    t_ver = kernel_us(verify)
    t_conv = kernel_us(conv)
    t_rb = kernel_us(rollback)
    t_rc = kernel_us(rollback_conv)

    # rollback by checkpoint and replay instead of capture: verify without H, then replay the accepted
    # prefix from the checkpoint S_in (the same step, timed the same way, on the same sets)
    def verify_nocap(d):
        gdn.verify(d["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"], None,
                   d["o"], wl.Hk)

    def replay(d):
        gdn.replay(d["accept"], d["y"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"],
                   wl.Hk, hist=d["hist"], win=d["win"])

    def replay_step(d):
        conv(d)
        verify_nocap(d)
        replay(d)

    t_ver_nocap = kernel_us(verify_nocap)
    t_replay = kernel_us(replay)
    t_replay_step = kernel_us(replay_step)

    vb = verify_bytes(wl)
    sb = step_bytes(wl)
    cpk = copy_peak(torch, dev)
    # the step's state bytes: the checkpoint, K-1 captured states and the final state
    state_out = wl.B * wl.Hv * wl.dv * wl.dk * 4 * (wl.T + 1)
    wpk = write_peak(torch, dev, step_bytes_=state_out, sets=R)
    if mode == "fused":
        # the dominant (and only) kernel of the step: gdn_verify_step
        dom, dom_bytes, dom_us = "gdn_verify_step", sb, t_fused
        sha = source_sha(*STEP_SOURCES)
    else:
        dom, dom_bytes, dom_us = "gdn_verify", vb, t_ver
        sha = source_sha(*VERIFY_SOURCES)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = read_traffic(dom, wl.name, sha)
    mean_rb_bytes = sum(rollback_bytes(wl, [a]) for a in accepts) / len(accepts)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "ms_per_step_trials": {"median": round(ms_per_step, 6), "min": round(min(trial_ms), 6),
                               "max": round(max(trial_ms), 6), "trials": len(trial_ms)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "B": wl.B, "K": wl.T, "Hk": wl.Hk, "Hv": wl.Hv, "dk": wl.dk, "dv": wl.dv,
            "C": wl.C, "conv_width": wl.W, "io_dtype": "bf16" if wl.bf16 else "f32", "state_dtype": "f32",
            "o_dtype": "f32" if args.o_f32 else "bf16",
            "step": {"three": "conv_step + verify(capture) + rollback",
                     "two": "rollback_conv_step (rollback of the previous window + conv_step, one launch) + "
                            "verify(capture)",
                     "fused": "verify_step: rollback of the previous window (start state and conv history picked "
                              "by its accept length) + conv_step + verify(capture), one launch"}[mode],
            "buffer_sets": R,
            "working_set_MB": round(R * set_bytes / 2 ** 20, 1), "launch": "eager" if args.eager else ("hip_graph, %d steps per graph" % per_graph),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "device_copy_GBs": cpk["GBs"],
            "frac_of_device_copy": round(achieved / cpk["GBs"], 4),
            "device_write_GBs": wpk["GBs"],
            "frac_of_device_write": round(achieved / wpk["GBs"], 4),
        },
        "detail": {
            "kernel": dom,
            "kernel_bytes_per_launch": dom_bytes,
            "kernel_us": round(dom_us, 3),
            "verify_step_us": round(t_fused, 3),
            "resident_step_us": None if t_resident is None else round(t_resident, 3),
            "resident_working_set_MB": round(2 * set_bytes / 2 ** 20, 1),
            "verify_step_bytes_per_launch": sb,
            "verify_bytes_per_launch": vb,
            "verify_us": round(t_ver, 3),
            # state traffic alone (the start state read, every state written; the fused step also writes
            # the checkpoint) over the kernel's duration
            "verify_state_GBs": round((wl.T + 1) * wl.B * wl.Hv * wl.dv * wl.dk * 4 / (t_ver * 1e-6) / 1e9, 1),
            "verify_step_state_GBs": round((wl.T + 2) * wl.B * wl.Hv * wl.dv * wl.dk * 4 / (t_fused * 1e-6) / 1e9, 1),
            "conv_us": round(t_conv, 3),
            "rollback_us": round(t_rb, 3),
            "rollback_conv_us": round(t_rc, 3),
            "checkpoint_replay": {"step_us": round(t_replay_step, 3), "verify_no_capture_us": round(t_ver_nocap, 3),
                                  "replay_us": round(t_replay, 3),
                                  "tokens_per_s": round(tokens / (t_replay_step * 1e-6), 1),
                                  "step": "conv_step + verify(no capture) + replay(accepted prefix) + conv rows"},
            "conv_GBs": round(conv_bytes(wl) / (t_conv * 1e-6) / 1e9, 1),
            "rollback_GBs": round(mean_rb_bytes / (t_rb * 1e-6) / 1e9, 1),
            "verify_only_tokens_per_s": round(tokens / (t_ver * 1e-6), 1),
            # tokens per second per layer counting the conv step and the verify (rollback apart)
            "conv_verify_tokens_per_s": round(tokens / ((t_conv + t_ver) * 1e-6), 1),
            "wall_ms_timed": round(wall_ms, 3),
            "settle": {"steps": settle_steps, "min_ms": args.settle_ms},
            "device_copy": cpk,
            "device_write": wpk,
            "o_dtype": "f32" if args.o_f32 else "bf16",
            "source_sha": sha,
            "accept_lengths": accepts,
        },
    }
    if not args.no_other_workloads:
        out["detail"]["other_workloads"] = other_workloads(torch, gdn, synth, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
