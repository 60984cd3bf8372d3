#!/usr/bin/env python3
"""Benchmark: one full distance-bound smoothing pass per step on one MI355X.

A step runs one pass (all rounds k = 0..n-1) through the C ABI, dbs_smooth,
on its own copy of the synthetic input, staged in HBM before the timed region
(the pass works in place; where the copies would take more than 96 GB a step
restores the input with a device copy inside the timed region instead).  The
default workload is n = 12288: 48 self-avoiding chains of 256 atoms packed in
a 90 A sphere (dense fp32 U and L, 1.2 GB together).

Printed: one JSON line with
  value        bound-updates/s = 2 n^3 batch / (seconds per step)
  executed_frac_of_fp32_peak  the operations the symmetric schedule
               executes (6 per (i,j,k) triple of the cells it keeps current)
               / t / 157.3e12, the MI355X fp32 vector peak
  dense_equivalent_frac_of_fp32_peak  = 6 n^3 batch / t / 157.3e12: the
               metric's dense count, about twice the executed work, so it can
               exceed 1
  roofline     the bulk phase-3 kernel (k_quads on 64x64 quadrants):
               executed ops of the cells a launch stores / mean launch time
               from HIP events (dbs_smooth_profiled on the launch stream),
               against the 157.3 T fp32 vector peak
  all_configs  the four smaller workloads: median GPU pass time, executed
               fraction of peak, the same pass replayed from a captured HIP
               graph, and the oracle's full pass on this host
  perk         the per-round kernel: HBM bytes of the round formulation
               (16 B per cell per round) / mean round time
  restraints   the workload's restraint list to dense bounds (fill + scatter)
  tightened    the mask of cells a pass changed
  directed     the same pass with sums rounded up and differences rounded
               down (sound bounds on inputs off the 2^-6 grid)
  packed       the same pass on the one-buffer layout (U above the diagonal,
               L below), with the pack and unpack steps timed apart
  cpu_baseline the CPU reference (oracle) on a bounded prefix of rounds of
               the same workload, on this host's cores
Run with --gpus N > 1 and it exits: the library has no multi-GPU path.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bound-updates/s (2·n³ per pass) + % fp32 VALU peak; HBM GB/s per-k kernel"
FP32_VALU_PEAK = 157.3e12       # MI355X fp32 vector, ops/s (an FMA counted as 2)
HBM_PEAK = 8.0e12               # MI355X HBM3E, bytes/s
OPS_PER_TRIPLE = 6              # 1 add + 1 min (upper), 2 sub + 2 max (lower)
TILE, BK = 128, 64              # blocked-path geometry (csrc/blocked.hip)
COUNTERS = os.path.join(ROOT, "profiles", "k_quads_n12288_counters.json")
# device memory the timed steps' staged input copies may take (288 GB of HBM)
STAGE_BYTES = 96 * 2**30
KERNEL_SRC = os.path.join(ROOT, "distance_geometry_bound_amd", "csrc", "blocked.hip")
ROUND_COUNTERS = os.path.join(ROOT, "profiles", "k_round_vec_n12288_counters.json")
VALU_COUNTERS = os.path.join(ROOT, "profiles", "k_quads_n12288_valu.json")
ROUND_SRC = os.path.join(ROOT, "distance_geometry_bound_amd", "csrc", "round.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="n12288",
                    choices=["n128", "n1024", "b64n500", "n4096", "n12288"])
    ap.add_argument("--algo", default="auto", choices=["auto", "blocked", "lds", "perk"])
    ap.add_argument("--perk-rounds", type=int, default=64,
                    help="rounds of the per-round kernel to time (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 = skip)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-steps-extra", dest="steps_extra", action="store_false",
                    help="skip timing the restraint-to-bounds and tightened-mask steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy 5 times (counter scale)")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the sweep over the smaller workloads")
    return ap.parse_args()


def copy_calibration():
    import torch

    dev = torch.device("cuda:0")
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_calibration_bytes": nbytes, "dispatches": 5}), flush=True)


def tiles_units_per_pass(n, batch, ahead, W):
    """(stored, dense) (i,j,k) triples of the bulk phase-3 launches over one pass.

    The pass steps over W k-blocks at a time (dbs_step_blocks).  The launch of
    the step starting at block K runs the step's atoms over the 64x64
    quadrants (A, B) of the TILE x TILE tiles with A <= B (the upper tiles'
    quadrants and the upper and diagonal ones of the diagonal tiles) and
    stores every cell outside the step's bands (final after its panel) and
    the bands of the `ahead` steps after it (updated ahead on the second
    stream; fewer near the end).  `stored` counts those cells x the launch's
    atoms; `dense` counts the full square of live rows x live columns (the
    cells below the diagonal follow by symmetry)."""
    TB = -(-n // BK)
    stored = dense = 0
    for K in range(0, TB, W):
        end = min(TB, K + W * (1 + ahead))
        r = [0 if K <= B < end else min(n, B * BK + BK) - B * BK for B in range(TB)]
        S, Q = sum(r), sum(x * x for x in r)
        atoms = min(n, (K + W) * BK) - K * BK
        stored += (S * S + Q) // 2 * atoms
        dense += S * S * atoms
    return stored * batch, dense * batch


def executed_triples(n, batch):
    """(i,j,k) triples the symmetric schedule executes in one pass: every
    cell of the 64x64 quadrants (A, B) with A <= B, for every atom k (phases
    1-2 repeat the diagonal tile's rounds per panel workgroup; those repeats
    are not counted)."""
    TB = -(-n // BK)
    rows = [min(n, (B + 1) * BK) - B * BK for B in range(TB)]
    return (n * n + sum(r * r for r in rows)) // 2 * n * batch


def source_digest(path):
    """sha256 of a C++ source with its // comments and all whitespace removed,
    so that the counter record stays valid across edits of comments only."""
    import re
    text = re.sub(r"//[^\n]*", "", open(path).read())
    return hashlib.sha256(re.sub(r"\s+", "", text).encode()).hexdigest()


def counters_traffic(n, batch, record=COUNTERS, source=KERNEL_SRC):
    """HBM bytes per launch of a kernel from its committed counter run (the
    phase-3 bulk by default), if the kernel source (comments aside) is
    unchanged since it was taken; else None."""
    try:
        rec = json.load(open(record))
    except (OSError, ValueError):
        return None
    sha = source_digest(source)
    if rec.get("source_sha256") != sha or rec.get("n") != n or rec.get("batch") != batch:
        return None
    return rec.get("traffic_bytes_per_launch")


def valu_counters(n, batch):
    """Per-clock VALU issue and the clock of the bulk launch, from the
    committed SQ/GRBM counter run, if the source is unchanged since; else None."""
    try:
        rec = json.load(open(VALU_COUNTERS))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(KERNEL_SRC) or rec.get("n") != n or \
            rec.get("batch") != batch:
        return None
    return {"valu_lanes_per_clk_per_simd": rec["valu_lanes_per_clk_per_simd"],
            "clock_ghz": rec["clock_ghz"],
            "sq_insts_valu_per_launch": rec["sq_insts_valu_per_launch"],
            "modelled_insts_per_launch": rec["modelled_insts_per_launch"]}


def extra_steps(W, U, L, U0, L0, dev, reps=3):
    """Time the steps around a pass on the same workload: the restraint list
    to dense bounds (placeholder fill + interval scatter; the fill writes 8
    bytes per cell) and the tightened-cell mask of a finished pass (reads 16,
    writes 1 byte per cell).  Both are HBM-bound."""
    import torch

    import distance_geometry_bound_amd as dgb
    from distance_geometry_bound_amd import gen

    res = {}
    mol, ia, ja, lo, hi, ul, uu, n, nb = gen.workload_restraints(W.name)
    t = [torch.from_numpy(x).to(dev) for x in (mol, ia, ja, lo, hi)]
    s = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dgb.bounds_from_restraints(n, t[1], t[2], t[3], t[4], ul, uu, mol=t[0], batch=nb,
                               out=(U, L))
    ms = 0.0
    for _ in range(reps):
        e0.record(s)
        _, _, st = dgb.bounds_from_restraints(n, t[1], t[2], t[3], t[4], ul, uu, mol=t[0],
                                              batch=nb, out=(U, L))
        e1.record(s)
        torch.cuda.synchronize(dev)
        ms += e0.elapsed_time(e1) / reps
    cells = n * n * nb
    res["restraints"] = {"count": int(len(ia)), "status": st, "ms": ms,
                         "GBps_fill": 8.0 * cells / (ms * 1e-3) / 1e9,
                         "frac_hbm": 8.0 * cells / (ms * 1e-3) / HBM_PEAK,
                         "bytes": 8 * cells}
    U.copy_(U0)
    L.copy_(L0)
    dgb.smooth(U, L)
    dgb.tightened(U0, L0, U, L)
    ms = 0.0
    for _ in range(reps):
        e0.record(s)
        m = dgb.tightened(U0, L0, U, L)
        e1.record(s)
        torch.cuda.synchronize(dev)
        ms += e0.elapsed_time(e1) / reps
    res["tightened"] = {"ms": ms, "cells_changed": int(m.sum().item()),
                        "GBps": 17.0 * cells / (ms * 1e-3) / 1e9,
                        "frac_hbm": 17.0 * cells / (ms * 1e-3) / HBM_PEAK}
    return res


def packed_pass(U0, L0, dev, reps=2):
    """Time the one-buffer layout on the same workload: pack (reads the one
    bound a cell keeps and writes it: 8 bytes per cell), one full pass in
    place on the packed buffer, unpack (reads P once and writes U and L: 12
    bytes per cell)."""
    import torch

    import distance_geometry_bound_amd as dgb

    s = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    P0 = dgb.pack(U0, L0)
    P = torch.empty_like(P0)
    P.copy_(P0)
    dgb.smooth_packed(P)                     # warm
    ms = [0.0, 0.0, 0.0]
    for _ in range(reps):
        P.copy_(P0)
        ev[0].record(s)
        dgb.pack(U0, L0, out=P)
        ev[1].record(s)
        dgb.smooth_packed(P)
        ev[2].record(s)
        dgb.unpack(P)
        ev[3].record(s)
        torch.cuda.synchronize(dev)
        for i in range(3):
            ms[i] += ev[i].elapsed_time(ev[i + 1]) / reps
    n, batch = U0.shape[-1], U0.numel() // (U0.shape[-1] ** 2)
    triples = float(n) ** 3 * batch
    cells = n * n * batch
    return {"pass_ms": ms[1], "value": 2.0 * triples / (ms[1] * 1e-3),
            "executed_frac_of_fp32_peak": OPS_PER_TRIPLE * executed_triples(n, batch)
            / (ms[1] * 1e-3) / FP32_VALU_PEAK,
            "dense_equivalent_frac_of_fp32_peak": OPS_PER_TRIPLE * triples / (ms[1] * 1e-3)
            / FP32_VALU_PEAK,
            "pack_ms": ms[0], "pack_GBps": 8.0 * cells / (ms[0] * 1e-3) / 1e9,
            "unpack_ms": ms[2], "unpack_GBps": 12.0 * cells / (ms[2] * 1e-3) / 1e9,
            "bytes": 4 * cells}


def directed_pass(U, L, U0, L0, dev, reps=2):
    """Time the directed-rounding pass on the same workload (the same kernels
    with the fp32 rounding mode set toward +inf)."""
    import torch

    import distance_geometry_bound_amd as dgb

    s = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    U.copy_(U0)
    L.copy_(L0)
    dgb.smooth_directed(U, L)                # warm
    ms = 0.0
    for _ in range(reps):
        U.copy_(U0)
        L.copy_(L0)
        e0.record(s)
        dgb.smooth_directed(U, L)
        e1.record(s)
        torch.cuda.synchronize(dev)
        ms += e0.elapsed_time(e1) / reps
    n, batch = U0.shape[-1], U0.numel() // (U0.shape[-1] ** 2)
    triples = float(n) ** 3 * batch
    return {"pass_ms": ms, "value": 2.0 * triples / (ms * 1e-3),
            "executed_frac_of_fp32_peak": OPS_PER_TRIPLE * executed_triples(n, batch)
            / (ms * 1e-3) / FP32_VALU_PEAK,
            "dense_equivalent_frac_of_fp32_peak": OPS_PER_TRIPLE * triples / (ms * 1e-3)
            / FP32_VALU_PEAK}


def cpu_baseline(W, target_s):
    """Time the oracle on a prefix of rounds of the same workload."""
    import ctypes

    import numpy as np

    import oracle

    lib = oracle.load()
    threads = oracle.max_threads()
    f32p = ctypes.POINTER(ctypes.c_float)
    U = np.array(W.U[:1], copy=True)
    L = np.array(W.L[:1], copy=True)

    def run(rounds):
        t0 = time.perf_counter()
        rc = lib.dbs_oracle_rounds(U.ctypes.data_as(f32p), L.ctypes.data_as(f32p), W.n, 1, 0,
                                   rounds, threads)
        dt = time.perf_counter() - t0
        assert rc == 0
        return dt

    # grow the prefix until it costs a quarter of the target, then scale
    rounds = 4
    t = run(rounds)
    while t < 0.25 * target_s and rounds < W.n:
        rounds = min(W.n, rounds * 4)
        t = run(rounds)
    rounds = int(max(1, min(W.n, round(rounds * target_s / max(t, 1e-6)))))
    t = run(rounds)
    bu = 2.0 * W.n * W.n * rounds
    return {"value": bu / t, "unit": "bound-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"rounds 0..{rounds - 1} of the {W.name} pass on molecule 0 "
                      f"({rounds} of {W.n} rounds, {t:.1f} s)",
            "seconds": t}


def config_sweep(names, dev, reps=15, oracle_on=True):
    """Each workload in `names`: the median device time of one full pass
    (HIP events on the launch stream, the input restored outside them), its
    executed fraction of the fp32 peak, the median time of the same pass
    replayed from a captured HIP graph (and whether its bits equal the eager
    pass's), and the oracle's full pass on this host's cores (wall time, one
    run)."""
    import numpy as np
    import torch

    import distance_geometry_bound_amd as dgb
    from distance_geometry_bound_amd import gen

    res = {}
    s = torch.cuda.current_stream(dev)
    for name in names:
        W = gen.make_workload(name)
        n, batch = W.n, W.batch
        U0 = torch.from_numpy(W.U).to(dev)
        L0 = torch.from_numpy(W.L).to(dev)
        U, L = torch.empty_like(U0), torch.empty_like(L0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        times = []
        for r in range(reps + 2):
            U.copy_(U0)
            L.copy_(L0)
            ev[0].record(s)
            dgb.smooth(U, L)
            ev[1].record(s)
            torch.cuda.synchronize(dev)
            if r >= 2:
                times.append(ev[0].elapsed_time(ev[1]))
        ms = float(np.median(times))
        ref_u, ref_l = U.clone(), L.clone()
        # the same pass captured once into a HIP graph and replayed (its own
        # stream; the input restored outside the events), which removes the
        # host's launch gaps between the pass's kernels
        gs = torch.cuda.Stream(dev)
        graph = torch.cuda.CUDAGraph()
        gtimes = []
        with torch.cuda.stream(gs):
            U.copy_(U0)
            L.copy_(L0)
            gs.synchronize()
            with torch.cuda.graph(graph, stream=gs):
                dgb.smooth(U, L)
            for r in range(reps + 2):
                U.copy_(U0)
                L.copy_(L0)
                ev[0].record(gs)
                graph.replay()
                ev[1].record(gs)
                gs.synchronize()
                if r >= 2:
                    gtimes.append(ev[0].elapsed_time(ev[1]))
        same = bool(torch.equal(U.view(torch.int32), ref_u.view(torch.int32)) and
                    torch.equal(L.view(torch.int32), ref_l.view(torch.int32)))
        del graph
        triples = float(n) ** 3 * batch
        entry = {"n": n, "batch": batch, "algo": dgb.auto_algo(n, batch),
                 "lookahead_bands": dgb.lookahead_bands(n, batch),
                 "pass_ms_median": ms, "pass_ms_min": float(min(times)), "reps": reps,
                 "value": 2.0 * triples / (ms * 1e-3),
                 "executed_frac_of_fp32_peak": OPS_PER_TRIPLE * executed_triples(n, batch)
                 / (ms * 1e-3) / FP32_VALU_PEAK,
                 "graph_replay_ms_median": float(np.median(gtimes)),
                 "graph_replay_same_bits": same}
        if oracle_on:
            import oracle
            t0 = time.perf_counter()
            oracle.smooth(W.U, W.L)
            t = time.perf_counter() - t0
            entry["oracle_full_pass_s"] = t
            entry["oracle_value"] = 2.0 * triples / t
            entry["oracle_cores"] = oracle.max_threads()
            entry["gpu_over_oracle"] = t / (ms * 1e-3)
        res[name] = entry
        print(f"[bench] {name}: {ms:.3f} ms per pass, {entry['graph_replay_ms_median']:.3f} ms "
              f"replayed from a graph", file=sys.stderr, flush=True)
        del U0, L0, U, L, ref_u, ref_l
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import distance_geometry_bound_amd as dgb
    from distance_geometry_bound_amd import gen

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    W = gen.make_workload(args.workload)
    n, batch = W.n, W.batch
    print(f"[bench] workload {W.name}: n={n} batch={batch} generated in "
          f"{time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    U0 = torch.from_numpy(W.U).to(dev)
    L0 = torch.from_numpy(W.L).to(dev)
    U = torch.empty_like(U0)
    L = torch.empty_like(L0)
    algo = args.algo if args.algo != "auto" else dgb.auto_algo(n, batch)

    # Every step smooths its own copy of the input, staged in HBM before the
    # timed region (the pass works in place); past STAGE_BYTES of copies a
    # step restores the input with a device copy instead.
    nstage = args.warmup + args.steps
    staged = nstage * 2 * U0.numel() * 4 <= STAGE_BYTES
    bufs = [(U0.clone(), L0.clone()) for _ in range(nstage)] if staged else []
    torch.cuda.synchronize(dev)

    def step(i):
        if staged:
            dgb.smooth(bufs[i][0], bufs[i][1], algo=algo)
            return
        U.copy_(U0)
        L.copy_(L0)
        dgb.smooth(U, L, algo=algo)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize(dev)
    del bufs
    dt = (time.perf_counter() - t0) / max(args.steps, 1)
    print(f"[bench] timed {args.steps} steps: {dt * 1e3:.2f} ms/step", file=sys.stderr, flush=True)
    triples = float(n) ** 3 * batch
    out = {
        "metric": METRIC,
        "value": 2.0 * triples / dt,
        "unit": "bound-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": W.name, "n": n, "batch": batch, "algo": algo,
                   "step": ("one full pass on a copy of the input staged in HBM" if staged
                            else "restore U,L (device copy) + one full pass")},
        "executed_frac_of_fp32_peak": OPS_PER_TRIPLE * executed_triples(n, batch) / dt
        / FP32_VALU_PEAK,
        "dense_equivalent_frac_of_fp32_peak": OPS_PER_TRIPLE * triples / dt / FP32_VALU_PEAK,
    }

    # per-kernel device times from HIP events around every launch of a pass
    prof_steps = max(1, min(args.steps, 3))
    tot = {k: [0, 0.0] for k in dgb.PROF_KINDS}
    for _ in range(prof_steps):
        U.copy_(U0)
        L.copy_(L0)
        p = dgb.smooth_profiled(U, L, algo=algo)
        for k, (c, ms) in p.items():
            tot[k][0] += c
            tot[k][1] += ms
    out["phases_ms_per_pass"] = {k: v[1] / prof_steps for k, v in tot.items() if v[0]}
    out["launches_per_pass"] = {k: v[0] // prof_steps for k, v in tot.items() if v[0]}
    if tot["tiles"][0]:
        launches = tot["tiles"][0] // prof_steps
        launch_ms = tot["tiles"][1] / tot["tiles"][0]
        ahead = dgb.lookahead_bands(n, batch)
        width = dgb.step_blocks(n, batch)
        stored, dense = tiles_units_per_pass(n, batch, ahead, width)
        ops = OPS_PER_TRIPLE * stored / launches          # per launch, averaged over the pass
        achieved = ops / (launch_ms * 1e-3)
        traffic = counters_traffic(n, batch)
        # algorithmic HBM bytes of a launch: read and write U and L of every
        # stored cell once (16 B), and read the step's panel rows once
        atoms = min(n, width * BK)
        alg_bytes = 16.0 * stored / launches / atoms + 8.0 * atoms * n * batch
        out["roofline"] = {
            "bound": "alu", "kernel": "k_quads (dense bulk of phase 3)",
            "achieved": achieved / 1e12, "peak": FP32_VALU_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": achieved / FP32_VALU_PEAK,
            "peak_basis": "MI355X fp32 vector peak; achieved counts the 6 fp32 add/sub/min/max "
                          "operations per (i,j,k) triple of the cells a launch stores",
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "launch_ms": launch_ms, "launches": tot["tiles"][0], "lookahead_bands": ahead,
            "step_blocks": width,
            "ops_per_launch": ops,
            "issue_counters": valu_counters(n, batch),
            "dense_equivalent_frac": OPS_PER_TRIPLE * dense / launches / (launch_ms * 1e-3)
                                     / FP32_VALU_PEAK,
        }

    if args.perk_rounds > 0:
        R = min(args.perk_rounds, n)
        U.copy_(U0)
        L.copy_(L0)
        s = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dgb.smooth_rounds(U, L, 0, 1)            # warm
        e0.record(s)
        dgb.smooth_rounds(U, L, 1, 1 + R if 1 + R <= n else n)
        e1.record(s)
        torch.cuda.synchronize(dev)
        R = min(R, n - 1)
        if R > 0:
            ms = e0.elapsed_time(e1) / R
            gbps = 16.0 * n * n * batch / (ms * 1e-3) / 1e9
            out["perk"] = {"kernel": "k_round_vec" if n % 4 == 0 else "k_round_scalar",
                           "rounds": R, "ms_per_round": ms, "GBps": gbps,
                           "frac_hbm": gbps * 1e9 / HBM_PEAK,
                           "bytes_per_round": 16 * n * n * batch,
                           "traffic": counters_traffic(n, batch, ROUND_COUNTERS, ROUND_SRC)}

    if args.steps_extra:
        out.update(extra_steps(W, U, L, U0, L0, dev))
        out["directed"] = directed_pass(U, L, U0, L0, dev)
        out["packed"] = packed_pass(U0, L0, dev)

    if not args.no_cpu and args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)

    if args.configs and W.name == "n12288":
        del U0, L0, U, L
        out["all_configs"] = config_sweep(("n128", "n1024", "b64n500", "n4096"), dev,
                                          oracle_on=not args.no_cpu)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
