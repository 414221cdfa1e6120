#!/usr/bin/env python3
"""Throughput benchmark of the shallow-water Roe step on one MI355X.

A "step" is one explicit time step of the whole hot path: Roe edge fluxes
with the bed term and pollutant transport, per-cell accumulation and CFL
wave speeds with the global dt minimum, and the conserved-variable update.

Default workload: the 4096 x 4096 structured grid (one layer + pollutant,
fp32, x periodic / y walls, seeded smooth flow over a 64-Gaussian bed),
500 steps per timed call.  Each of `repeats` timed batches uploads W^0
(outside the timed region), runs `warmup` untimed steps (the first of them
pays the one-off dt pass of the uploaded state), then times one
swe_step(K) call -- steps warmup+1 .. warmup+K of the workload -- bracketed by
HIP events recorded on the context's stream; the median is reported.

Prints ONE JSON line with the metric, a roofline object for the dominant
kernel and the CPU oracle timed on this host on a bounded sample.
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

PEAK_HBM_GBS = 8000.0
WORKLOADS = {
    "dam-break-64": "one-layer SWE + pollutant, 64x64 structured, 1 m cells, flat bed, dam break, walls, fp64",
    "hump-1024": "one-layer SWE + pollutant, 1024x1024 structured, 1 m cells, 16-Gaussian bed, Gaussian hump, walls",
    "flow-4096": "one-layer SWE + pollutant, 4096x4096 structured, 10 m cells, 64-Gaussian bed, smooth flow, "
                 "periodic x / walls y, fp32",
    "tri-2M": "one-layer SWE, 2M-triangle jittered Morton-ordered mesh, circular dam break, walls, fp64",
    "two-layer-1M": "two-layer SWE (IR-Roe 4x4), 1M-triangle jittered mesh, internal dam break, walls, fp64",
}
# the precision each workload runs in unless --precision says otherwise
PRECISION = {"dam-break-64": "f64", "hump-1024": "f64", "flow-4096": "f32", "tri-2M": "f64", "two-layer-1M": "f64"}
PROFILE_DIR = os.path.join(ROOT, "profiles")


def alg_bytes_per_cell(w, prec, E=None):
    """Algorithmic bytes per cell-update: read W^n and the bed, write W^{n+1};
    triangle meshes also read per-cell area and the edge list (two int32
    cell ids, normal x/y and length per edge)."""
    s = 4 if prec == "f32" else 8
    nv = w.nvars
    if w.kind == "cart":
        return (2 * nv + 1) * s
    return (2 * nv + 2) * s + (E / w.ncells) * (8 + 3 * s)


def _code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed
    (string and character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


# The sources that make each kernel family: its own file, the mesh
# preprocessing it consumes, the shared device headers and the host code that
# picks its launch shape.
_KERNEL_SOURCES = {"k_cart": ("kern_cart.hip",), "k_tri": ("kern_tri.hip", "mesh_host.cpp"),
                   "k_edge": ("kern_edge.hip", "mesh_host.cpp")}


def kernel_source_hash(path, kernel=None):
    """Hash of the code (comments and layout ignored) that builds `kernel`
    (all of the library if None): counter records taken on other code are not
    reused."""
    h = hashlib.sha256()
    csrc = os.path.join(path, "finite_volume_shallow_amd", "csrc")
    own = None
    if kernel is not None:
        fam = next((k for k in _KERNEL_SOURCES if kernel.startswith(k)), None)
        if fam is None:
            raise ValueError(f"no source list for kernel {kernel}")
        own = _KERNEL_SOURCES[fam]
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".hpp", ".cpp")):
            continue
        if own is not None and f.startswith("kern_") and f not in own:
            continue
        if own is not None and f.endswith(".cpp") and f not in own:
            continue
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, prec, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except Exception:
        return None
    rec = data.get(f"{kernel}@{workload}-{prec}")
    if not rec or rec.get("src_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def _pmc_mean(csv_path, kernel_substr, counter):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} in {csv_path}")
    return sum(vals) / len(vals), len(vals)


def ingest_pmc(args):
    """Turn four rocprofv3 --pmc CSVs into HBM bytes per launch of a kernel.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel are scaled by
    bytes_known / counter of a plain device copy of known size, so that the
    result is in actual bytes moved; stored in profiles/traffic.json with the
    hash of the kernel sources the counters were taken on."""
    kf, kw, cf, cw = args.ingest_pmc
    kern = args.ingest_kernel
    copy_bytes = int(args.ingest_copy_gib * (1 << 30))
    f_k, n_f = _pmc_mean(kf, kern, "FETCH_SIZE")
    w_k, n_w = _pmc_mean(kw, kern, "WRITE_SIZE")
    f_c, _ = _pmc_mean(cf, "copyBuffer", "FETCH_SIZE")
    w_c, _ = _pmc_mean(cw, "copyBuffer", "WRITE_SIZE")
    f_scale = copy_bytes / (f_c * 1024.0)
    w_scale = copy_bytes / (w_c * 1024.0)
    rd = f_k * 1024.0 * f_scale
    wr = w_k * 1024.0 * w_scale
    path = os.path.join(PROFILE_DIR, "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    prec = args.precision or PRECISION[args.workload]
    key = f"{args.ingest_name}@{args.workload}-{prec}"
    data[key] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                 "fetch_scale": f_scale, "write_scale": w_scale,
                 "dispatches": [n_f, n_w], "src_hash": kernel_source_hash(ROOT, args.ingest_name)}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    json.dump(data, open(path, "w"), indent=1, sort_keys=True)
    print(json.dumps({key: data[key]}))


def _oracle_rate(src, nthreads, budget_s, max_steps):
    """Oracle cell-updates/s with nthreads threads: a one-step run, a two-step
    run for the per-step time, then a run of about budget_s seconds; the rate
    is taken from the difference with the one-step run, so that the oracle's
    one-off mesh setup does not count."""
    import oracle

    def timed(n):
        t0 = time.perf_counter()
        oracle.run(src, nsteps=n, nthreads=nthreads)
        return time.perf_counter() - t0

    t1 = timed(1)
    per_step = max(timed(2) - t1, 1e-4)
    steps = max(2, min(max_steps, 1 + int(budget_s / per_step)))
    tn = timed(steps)
    return src.ncells * (steps - 1) / max(tn - t1, 1e-9), steps, tn, t1


def cpu_baseline(w, prec, budget_s, gpu_value):
    """The oracle as it stands, on this host's cores, on the first steps of
    the same workload: one leg on all host threads (at most 16, the CPU share
    of one GPU) and one on a single thread, each about budget_s / 2 seconds of
    CPU work.  Reported as a baseline, with the GPU/oracle ratios; the pages'
    own speed-ups are quoted as context only (other hardware, precision and
    workload)."""
    import inputs
    nthreads = max(1, min(16, os.cpu_count() or 1))
    src = inputs.round_to_f32(w) if prec == "f32" else w
    rate, steps, tn, t1 = _oracle_rate(src, nthreads, budget_s / 2, w.nsteps)
    rate1, steps1, tn1, t11 = _oracle_rate(src, 1, budget_s / 2, w.nsteps)
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": rate, "unit": "cell-updates/s", "cores": nthreads, "kind": "oracle",
            "sample": f"steps 2..{steps} of the same workload ({w.ncells} cells), fp64 oracle, "
                      f"{tn:.1f} s for {steps} steps minus {t1:.1f} s for the first; "
                      f"{nthreads} OpenMP threads of {os.cpu_count()} logical CPUs ({model})",
            "single_thread": {"value": rate1, "unit": "cell-updates/s", "cores": 1,
                              "sample": f"steps 2..{steps1}, {tn1:.1f} s minus {t11:.1f} s for the first"},
            "gpu_over_oracle": {"threads": round(gpu_value / rate, 1), "single_thread": round(gpu_value / rate1, 1)},
            "context": "the pages' single-GPU IR-Roe speed-ups for big meshes (Tesla C2050 against "
                       "their CPU versions, precision not stated): 32x over one core, 10x over four "
                       "cores; not comparable with these figures"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="flow-4096", choices=list(WORKLOADS))
    ap.add_argument("--precision", choices=["f32", "f64"], default=None)
    ap.add_argument("--path", choices=["auto", "edge", "recompute"], default="auto",
                    help="kernel path: the fused kernels (auto), the explicit-edge path, or the fused "
                         "kernel with every cell evaluating all its edges (recompute, an ablation)")
    ap.add_argument("--entropy-fix", action="store_true",
                    help="with the Harten-Hyman entropy fix (one layer)")
    ap.add_argument("--scheme", choices=["ir", "classical"], default="ir",
                    help="numerical flux: IR-Roe (default) or the classical Roe flux")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed batches of --steps steps each, every one from W^0 after the untimed warmup "
                         "steps; the median is reported")
    ap.add_argument("--cpu-budget", type=float, default=24.0,
                    help="seconds of oracle work for the CPU baseline (half on all threads, half on one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-ref", type=float, default=0.0, metavar="GIB",
                    help="instead of the benchmark: time a plain device copy of GIB GiB "
                         "(the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--ingest-pmc", nargs=4, metavar=("KERN_FETCH", "KERN_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="instead of the benchmark: record HBM bytes per launch from rocprofv3 "
                         "counter CSVs into profiles/traffic.json")
    ap.add_argument("--ingest-kernel", default="k_cart_fused")
    ap.add_argument("--ingest-name", default="k_cart_fused")
    ap.add_argument("--ingest-copy-gib", type=float, default=1.0)
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the sharding design is described, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import finite_volume_shallow_amd as swe
    import inputs

    torch.cuda.set_device(0)
    if args.copy_ref > 0:
        n = int(args.copy_ref * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        reps = 5
        ev0.record()
        for _ in range(reps):
            dst.copy_(src)
        ev1.record()
        ev1.synchronize()
        ms = ev0.elapsed_time(ev1) / reps
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "ms": ms,
                          "GBps_read_plus_write": 8 * n / (ms / 1e3) / 1e9}), flush=True)
        return
    w = inputs.make_workload(args.workload)
    w.scheme = args.scheme
    w.entropy_fix = int(args.entropy_fix)
    prec = args.precision or w.precision
    K = args.steps or w.nsteps
    stream = torch.cuda.Stream()
    path = {"auto": swe.SWE_PATH_AUTO, "edge": swe.SWE_PATH_EDGE, "recompute": swe.SWE_PATH_RECOMPUTE}[args.path]
    desc, keep = swe.desc_from_workload(w, path=path, stream=stream, precision=prec)
    ctx = swe.swe_create_mesh(desc)
    del keep
    used_path = {swe.SWE_PATH_FUSED: "fused", swe.SWE_PATH_EDGE: "edge",
                 swe.SWE_PATH_RECOMPUTE: "recompute"}[swe.swe_path(ctx)]
    launch_shape = swe.swe_describe(ctx)

    times, one = [], []
    for _ in range(max(1, args.repeats)):
        # every timed batch is the same stretch of the simulation: W^0, the
        # warmup steps untimed (with the dt pass of the uploaded state), then
        # K steps timed
        swe.swe_set_state(ctx, w.z, w.state)
        if args.warmup:
            swe.swe_step(ctx, args.warmup, w.cfl)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        t_adv, _ = swe.swe_step(ctx, K, w.cfl)
        ev1.record(stream)
        ev1.synchronize()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1)
        times.append(ms)
        # one more call of a single step, timed the same way: its time is the
        # call's fixed part (batch set-up, read-back, return) plus one launch,
        # so (T_K - T_1) / (K - 1) is the average duration of one step's launch
        if K > 1:
            ev2 = torch.cuda.Event(enable_timing=True)
            ev3 = torch.cuda.Event(enable_timing=True)
            ev2.record(stream)
            swe.swe_step(ctx, 1, w.cfl)
            ev3.record(stream)
            ev3.synchronize()
            one.append(ev2.elapsed_time(ev3))
    swe.swe_destroy(ctx)

    N = w.ncells
    times.sort()
    med = times[len(times) // 2]  # median batch
    value = N * K / (med / 1e3)
    ms_step = med / K
    # average launch duration of the step kernel (live, from the K-step and
    # 1-step calls); the per-step time of the whole call when K = 1
    if one:
        one.sort()
        ms_launch = max((med - one[len(one) // 2]) / (K - 1), 1e-6)
    else:
        ms_launch = ms_step
    E = None
    if w.kind == "tri":
        # edges of a triangle mesh: (3 N + boundary) / 2, counted from the mesh
        import numpy as np
        t = w.tri
        e = np.sort(np.stack([t, np.roll(t, -1, axis=1)], axis=2).reshape(-1, 2), axis=1)
        E = int(np.unique(e, axis=0).shape[0])
    bpc = alg_bytes_per_cell(w, prec, E)
    if used_path != "edge":
        # one-layer triangle meshes of regular size run the pipelined kernel
        kernel = "k_cart_fused" if w.kind == "cart" else ("k_tri_pipe" if w.nlayers == 1 else "k_tri_fused")
        if used_path == "recompute":  # one workgroup per block on triangles
            kernel = ("k_cart_fused" if w.kind == "cart" else "k_tri_fused") + "-recompute"
    else:
        kernel = "k_edge_flux+k_cell_dt+k_cell_update"
    # one fused launch per step: algorithmic bytes of a step over the average
    # launch duration
    achieved = bpc * N / (ms_launch / 1e3) / 1e9
    src_hash = kernel_source_hash(ROOT, kernel)
    # counters are recorded per kernel instance: the classical-flux kernel is
    # another instance (its own name in the traffic table)
    variant = ("-classical" if args.scheme == "classical" else "") + ("-hh" if args.entropy_fix else "")
    traffic = measured_traffic(kernel + variant, args.workload, prec, src_hash)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": kernel, "alg_bytes_per_cell": bpc, "src_hash": src_hash,
                "launch_us": round(ms_launch * 1e3, 2),
                "launch_from": "(T(K steps) - T(1 step)) / (K - 1), HIP events on the context stream"}
    out = {
        "metric": "cell-updates/sec per Roe time step",
        "value": value,
        "unit": "cell-updates/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}"
                               + (" (classical Roe flux)" if args.scheme == "classical" else "")
                               + (" (Harten-Hyman entropy fix)" if args.entropy_fix else ""), "cells": N,
                   "scheme": args.scheme, "entropy_fix": bool(args.entropy_fix),
                   "precision": prec, "path": used_path, "kernel": launch_shape,
                   "simulated_seconds": t_adv},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, prec, args.cpu_budget, value)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
