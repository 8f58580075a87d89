"""Phase timelines of the fused verify step (gdn_verify_step) and of the chunked prefill.

    python -m speculative_verify_gdn_amd.build --timeline
    python -m speculative_verify_gdn_amd.timeline [--launches 6] [--sets 12] [--workload verify16|batched]
    python -m speculative_verify_gdn_amd.timeline --workload prefill [--launches 2]

Loads libgdn_timeline.so (the library built with the wall-clock marks of
csrc/gdn_timeline.h) and runs the step chained over buffer sets as bench.py
does (set r continues from set r-1's window; the sets together exceed the
Infinity Cache).  After warm-up, each measured launch runs alone: the marks
are cleared, one step is launched and synchronised, and the marks are read.
Marks (every wave, 100 MHz real-time counter; a wave keeps its marks in registers and writes
them once at its end, so the marks add no memory operations to the waits they measure):
  8 entry      the wave's first instruction (before the kernel arguments are read)
  0 start      the accept-length load issued
  5 accept     the accept length has arrived
  6 state      the start state has arrived (issued after the accept length)
  7 gates_v    the gates and the v conv are done
  1 conv0      the first chunk's q|k conv done, the checkpoint store issued
  2 barrier    past the first barrier (the recurrence may start)
  3 store0     the first state (H_0) store issued
  4 end        the wave's last store issued
Printed: one JSON line per launch with [min, p10, median, p90, max] of every
mark in microseconds after the launch's earliest entry, the median entry and
end per XCD (workgroup index mod 8), the end of the slowest wave, and per wave
role (waves 0-3 the first chunk's q|k conv, 4-6 the gates, 7-9 the v conv,
10-11 none) the medians of the marks before the first barrier.

With --workload prefill the marks are those of gdn_prefill_chunked's eleventh chunk
(chunk index 10) in every workgroup (the dk = 128, chunk 64 kernel), for the 4 state
waves and the 4 preparation waves: 0 chunk start, 1 phase-1 work done, 2 past the
phase-1 barrier, 3 phase-2 work done, 4 past the phase-2 barrier.  Printed: per role and per preparation
wave, the median and p90 over workgroups of each mark in nanoseconds after the
wave's own chunk start.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from speculative_verify_gdn_amd import gdn, synth  # noqa: E402

TL_GROUPS, TL_WAVES, TL_MARKS = 2048, 16, 16
NAMES = {8: "entry", 0: "start", 5: "accept", 6: "state", 7: "gates_v", 1: "conv0", 2: "barrier", 3: "store0", 4: "end"}


def prefill_timeline(lib, launches):
    lib.gdn_timeline_c64_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.gdn_timeline_c64_read.restype = ctypes.c_int
    lib.gdn_timeline_c64_clear.restype = ctypes.c_int
    wl = synth.WORKLOADS["prefill"]
    dev = torch.device("cuda", 0)
    inp = synth.make_inputs(wl, seed=0)
    d = {k: v.to(dev) for k, v in inp.items()}
    d["qkv"] = synth.make_qkv(wl, seed=0).to(dev)
    d["S_out"] = torch.empty_like(d["S_in"])
    d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=torch.bfloat16)

    def pre():
        gdn.prefill_chunked(d["qkv"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_in"], d["S_out"],
                            d["o"], wl.Hk, chunk=wl.chunk)

    for _ in range(3):
        pre()
    torch.cuda.synchronize()
    grid = wl.B * wl.Hv
    buf = np.zeros(TL_GROUPS * TL_WAVES * TL_MARKS, dtype=np.uint64)
    names = ("start", "p1_work", "p1_barrier", "p2_work", "p2_barrier")
    for n in range(launches):
        assert lib.gdn_timeline_c64_clear() == 0
        torch.cuda.synchronize()
        pre()
        torch.cuda.synchronize()
        assert lib.gdn_timeline_c64_read(buf.ctypes.data, buf.nbytes) == 0
        t = buf.reshape(TL_GROUPS, TL_WAVES, TL_MARKS)[:grid, :8, :].astype(np.int64)
        rel = (t - t[:, :, :1]) * 10   # 100 MHz ticks -> ns after the wave's own chunk start
        out = {"launch": n, "chunk": 10}
        for role, ws in (("state_waves", slice(0, 4)), ("prep_waves", slice(4, 8))):
            x = rel[:, ws, :]
            out[role] = {nm: [int(np.median(x[:, :, k])), int(np.percentile(x[:, :, k], 90))]
                         for k, nm in enumerate(names) if k}
        out["prep_wave_p1_work_median"] = [int(np.median(rel[:, 4 + w, 1])) for w in range(4)]
        out["prep_wave_p2_work_median"] = [int(np.median(rel[:, 4 + w, 3] - rel[:, 4 + w, 2])) for w in range(4)]
        out["state_wave_p2_work_median"] = [int(np.median(rel[:, w, 3] - rel[:, w, 2])) for w in range(4)]
        # finer marks (ns after the chunk start, median over workgroups and waves of the role)
        fine = {"prep": {5: "q|k arrived", 6: "operands + K^T written", 7: "norms written", 8: "gates scanned",
                         9: "gate factors written", 10: "diagonal block scaled", 11: "inverse written",
                         12: "gram tiles written"},
                "state": {15: "P, R done", 13: "U_0, U_1, O_0, O_1, first S update", 14: "phase 2 done"}}
        for role, ws in (("state", slice(0, 4)), ("prep", slice(4, 8))):
            x = rel[:, ws, :]
            out[role + "_marks"] = {nm: int(np.median(x[:, :, k])) for k, nm in fine[role].items()}
        print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--launches", type=int, default=6)
    ap.add_argument("--sets", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="verify16", help="verify16, batched (B=32, K=8) or prefill")
    args = ap.parse_args()
    lib = gdn.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn_timeline.so"))
    if args.workload == "prefill":
        prefill_timeline(lib, args.launches)
        return
    lib.gdn_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.gdn_timeline_read.restype = ctypes.c_int
    lib.gdn_timeline_clear.restype = ctypes.c_int
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)

    def make_set(seed):
        inp = synth.make_inputs(wl, seed=seed)
        d = {k: v.to(dev) for k, v in inp.items()}
        d["win"] = torch.empty(wl.B, wl.W - 1 + wl.T, wl.C, dtype=d["x"].dtype, device=dev)
        d["S_out"] = torch.empty_like(d["S_in"])
        d["H"] = torch.empty(wl.B, wl.T - 1, wl.Hv, wl.dv, wl.dk, device=dev)
        d["o"] = torch.empty(wl.B, wl.T, wl.Hv, wl.dv, device=dev, dtype=torch.bfloat16)
        d["S_ckpt"] = torch.empty_like(d["S_in"])
        return d

    sets = [make_set(r) for r in range(args.sets)]

    def step(r, first=False):
        d = sets[r % len(sets)]
        if first:
            gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_out"], d["H"],
                            d["o"], wl.Hk, S_in=d["S_in"], hist=d["hist"], S_ckpt=d["S_ckpt"], win=d["win"])
            return
        pv = sets[(r - 1) % len(sets)]
        gdn.verify_step(d["x"], d["w"], d["beta_raw"], d["alpha"], d["dt_bias"], d["A_log"], d["S_out"], d["H"],
                        d["o"], wl.Hk, prev=(pv["accept"], pv["S_ckpt"], pv["H"], pv["S_out"], pv["win"]),
                        S_ckpt=d["S_ckpt"], win=d["win"])

    for r in range(len(sets)):
        step(r, first=True)
    for r in range(args.warmup):
        step(r)
    torch.cuda.synchronize()
    grid = min((wl.dv // 8) * (wl.Hv // 3) * wl.B, TL_GROUPS)   # workgroups with marks
    nw = 12
    buf = np.zeros(TL_GROUPS * TL_WAVES * TL_MARKS, dtype=np.uint64)
    for n in range(args.launches):
        assert lib.gdn_timeline_clear() == 0
        torch.cuda.synchronize()
        step(args.warmup + n)
        torch.cuda.synchronize()
        assert lib.gdn_timeline_read(buf.ctypes.data, buf.nbytes) == 0
        t = buf.reshape(TL_GROUPS, TL_WAVES, TL_MARKS)[:grid, :nw].astype(np.int64)
        st = t[:, :, 8]
        t0 = st[st > 0].min()
        out = {"launch": n}
        for k, nm in NAMES.items():
            v = t[:, :, k]
            v = (v[v > 0] - t0) * 0.01   # 100 MHz -> us
            if v.size:
                out[nm] = [round(float(q), 2) for q in (v.min(), np.percentile(v, 10), np.median(v),
                                                        np.percentile(v, 90), v.max())]
        end = np.where(t[:, :, 4] > 0, (t[:, :, 4] - t0) * 0.01, np.nan).max(axis=1)   # per workgroup
        ent = np.where(t[:, :, 8] > 0, (t[:, :, 8] - t0) * 0.01, np.nan).min(axis=1)
        out["entry_median_by_xcd"] = [round(float(np.nanmedian(ent[x::8])), 2) for x in range(8)]
        out["end_median_by_xcd"] = [round(float(np.nanmedian(end[x::8])), 2) for x in range(8)]
        out["last_end"] = round(float(np.nanmax(end)), 2)
        # per wave role (waves 0-3 the first chunk's q|k conv, 4-6 the gates, 7-9 the v conv, 10-11
        # none): the median of each mark before the first barrier
        roles = (("conv0", slice(0, 4)), ("gates", slice(4, 7)), ("v", slice(7, 10)), ("idle", slice(10, 12)))
        out["by_role"] = {}
        for rn, ws in roles:
            x = t[:, ws, :]
            out["by_role"][rn] = {NAMES[k]: round(float(np.median((x[:, :, k][x[:, :, k] > 0] - t0) * 0.01)), 2)
                                  for k in (5, 6, 7, 1, 2) if (x[:, :, k] > 0).any()}
        # per workgroup: from its first wave's entry to its last wave's end
        dur = end - ent
        out["workgroup_span"] = [round(float(q), 2) for q in (np.nanmin(dur), np.nanmedian(dur), np.nanmax(dur))]
        print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
