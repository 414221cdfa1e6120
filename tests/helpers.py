"""Shared test helpers: run a workload through the GPU library or the oracle
and compare the two with the error measure the tolerances are stated in."""
from __future__ import annotations

import math
import sys

import numpy as np

import inputs
import oracle

FP64_TOL = 1e-10      # max relative error per field, fp64 runs
FP32_TOL = 1e-4       # max relative error per field after 100 steps, fp32


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def field_errors(got, ref, g=9.81):
    """Per conserved field: max_i |got - ref| / max_i |ref|.  A field that is
    identically zero in the reference is measured against the momentum scale
    max(h) * sqrt(g max(h)) instead."""
    hmax = max(float(np.abs(ref[0]).max()), 1e-300)
    fallback = hmax * math.sqrt(g * hmax)
    out = []
    for a, b in zip(got, ref):
        scale = float(np.abs(b).max())
        if scale == 0.0:
            scale = fallback
        out.append(float(np.abs(np.asarray(a) - np.asarray(b)).max()) / scale)
    return out


def gpu_run(w, nsteps=None, path=0, precision=None, stream=None):
    """Run a workload on the GPU through the C ABI.  Returns (state, dts, t)."""
    import finite_volume_shallow_amd as swe
    nsteps = w.nsteps if nsteps is None else nsteps
    desc, keep = swe.desc_from_workload(w, path=path, precision=precision, stream=stream)
    ctx = swe.swe_create_mesh(desc)
    try:
        swe.swe_set_state(ctx, w.z, w.state)
        t, last = swe.swe_step(ctx, nsteps, w.cfl)
        dts = swe.swe_get_dt_history(ctx)
        st = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    del keep
    return st, dts, t


def oracle_reference(w, nsteps=None, precision=None, chunk=None):
    """Oracle run on the inputs the GPU actually starts from (float32-rounded
    for a float32 run).  With ``chunk``, the run is taken ``chunk`` steps at
    a time (each piece restarts from the state the previous one left, so the
    result is the same) and a progress line is printed after each piece."""
    prec = precision or w.precision
    src = inputs.round_to_f32(w) if prec == "f32" else w
    nsteps = w.nsteps if nsteps is None else nsteps
    if not chunk or chunk >= nsteps:
        st, dts, _ = oracle.run(src, nsteps=nsteps)
        return st, dts
    parts, done, cur = [], 0, src
    while done < nsteps:
        k = min(chunk, nsteps - done)
        st, dts, _ = oracle.run(cur, nsteps=k)
        parts.append(dts)
        done += k
        say(f"    oracle: {done}/{nsteps} steps")
        cur = cur.copy(state=st)
    return st, np.concatenate(parts)


_ORACLE_CACHE = {}


def oracle_reference_cached(key, w, nsteps, precision, chunk=None):
    """oracle_reference, remembered under ``key`` for the rest of the test
    session (a long run that several tests compare against is taken once)."""
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = oracle_reference(w, nsteps=nsteps, precision=precision, chunk=chunk)
    st, dts = _ORACLE_CACHE[key]
    return [np.array(a, copy=True) for a in st], np.array(dts, copy=True)


def fsum(a):
    return math.fsum(np.asarray(a, dtype=float).tolist())


def tri_areas(w):
    p = w.node_xy[w.tri]
    return 0.5 * ((p[:, 1, 0] - p[:, 0, 0]) * (p[:, 2, 1] - p[:, 0, 1])
                  - (p[:, 2, 0] - p[:, 0, 0]) * (p[:, 1, 1] - p[:, 0, 1]))
