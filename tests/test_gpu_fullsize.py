"""GPU runs at the workloads' full sizes.

* Parity with the oracle, every cell, at full size: configs 1, 2 (fp64, all
  1000 steps), 2 and 3 in fp32 (100 steps, the fp32 parity point), 3 in
  fp64 (20 steps), 4 (all 200 steps) and 5 (all 200 steps; the two-layer
  oracle takes about a second per step there, so it runs in pieces with a
  progress line each).
* Full step counts on the GPU with properties that hold at any size: all
  values finite, depths positive, water, pollutant and layer masses
  conserved.
* The classical Roe flux, the Harten-Hyman entropy fix and the recomputed-
  edge organisation at the 4096^2, 2M-triangle and two-layer sizes.
"""
import numpy as np
import pytest

import inputs
from helpers import (FP32_TOL, FP64_TOL, field_errors, fsum, gpu_run,
                     oracle_reference, oracle_reference_cached, say, tri_areas)

pytestmark = pytest.mark.gpu

FULL = {
    "dam-break-64x64-f64": (lambda: inputs.dam_break(), "f64", 100),
    "hump-1024-f64": (lambda: inputs.gaussian_hump(), "f64", 1000),
    "hump-1024-f32": (lambda: inputs.gaussian_hump(), "f32", 100),
    "flow-4096-f32": (lambda: inputs.smooth_flow(), "f32", 100),
    # the float64 instance of the grid's streaming mode at its full size (20
    # steps: 3.4e8 oracle cell-updates)
    "flow-4096-f64": (lambda: inputs.smooth_flow(), "f64", 20),
    "tri-2M-f64": (lambda: inputs.circular_dam_break(), "f64", 200),
    "two-layer-1M-f64": (lambda: inputs.two_layer_dam_break(), "f64", 200),
}

# oracle runs of this length are taken in pieces of this many steps (with a
# progress line after each) and, for the two-layer mesh, shared by the tests
# that compare against the same reference run
CHUNK = 25


@pytest.mark.parametrize("name", list(FULL))
def test_fullsize_parity(name):
    make, prec, nsteps = FULL[name]
    w = make()
    say(f"[full parity] {name} cells={w.ncells} steps={nsteps}")
    got, dts, t = gpu_run(w, nsteps=nsteps, precision=prec)
    say("    gpu done; oracle running")
    if w.nlayers == 2:
        ref, rdts = oracle_reference_cached(("two-layer-1M", "ir", nsteps, prec), w, nsteps, prec, chunk=CHUNK)
    else:
        ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    errs = field_errors(got, ref, w.g)
    say(f"    field errors {['%.2e' % e for e in errs]}")
    assert max(errs) <= (FP64_TOL if prec == "f64" else FP32_TOL), errs
    dtol = 1e-12 if prec == "f64" else 1e-5
    derr = np.abs(dts - rdts).max() / rdts.max()
    say(f"    dt error {derr:.2e}")
    assert derr <= dtol


LONG = {
    "hump-1024-f32-1000": (lambda: inputs.gaussian_hump(), "f32", 1000),
    "flow-4096-f32-500": (lambda: inputs.smooth_flow(), "f32", 500),
    "flow-4096-f64-500": (lambda: inputs.smooth_flow(), "f64", 500),
    "two-layer-1M-200": (lambda: inputs.two_layer_dam_break(), "f64", 200),
}


@pytest.mark.parametrize("name", list(LONG))
def test_fullsize_full_length_properties(name):
    make, prec, nsteps = LONG[name]
    w = make()
    say(f"[full length] {name} cells={w.ncells} steps={nsteps}")
    got, dts, t = gpu_run(w, nsteps=nsteps, precision=prec)
    assert dts.shape == (nsteps,) and (dts > 0).all() and np.isfinite(dts).all()
    for a in got:
        assert np.isfinite(a).all()
    depth_vars = (0, 3) if w.nlayers == 2 else (0,)
    for v in depth_vars:
        assert got[v].min() > 0
    area = tri_areas(w) if w.kind == "tri" else np.full(w.ncells, w.dx * w.dy)
    init = inputs.round_to_f32(w) if prec == "f32" else w
    mass_vars = (0, 3) if (w.nlayers == 2 or w.ntracers) else (0,)
    tol = 1e-12 if prec == "f64" else 2e-5
    for v in mass_vars:
        m0 = fsum(init.state[v] * area)
        m1 = fsum(got[v] * area)
        say(f"    var {v}: relative mass change {abs(m1 - m0) / m0:.2e}")
        assert abs(m1 - m0) <= tol * m0


# The flux variants and the recomputation organisation at the headline sizes
# and in the launch shapes the benchmark times, every cell against the
# oracle.  The recomputed-edge path computes the same method as the shared-
# edge one, so its reference is the IR-Roe oracle run.
def _variant(make, scheme="ir", fix=0):
    def build():
        w = make()
        w.scheme = scheme
        w.entropy_fix = fix
        return w
    return build


VARIANTS = {
    "flow-4096-f32-classical": (_variant(inputs.smooth_flow, "classical"), "f32", 100, 0),
    "flow-4096-f32-entropy-fix": (_variant(inputs.smooth_flow, fix=1), "f32", 100, 0),
    "flow-4096-f32-recompute": (_variant(inputs.smooth_flow), "f32", 100, 3),
    "tri-2M-f64-classical": (_variant(inputs.circular_dam_break, "classical"), "f64", 200, 0),
    "tri-2M-f64-entropy-fix": (_variant(inputs.circular_dam_break, fix=1), "f64", 200, 0),
    "tri-2M-f64-recompute": (_variant(inputs.circular_dam_break), "f64", 200, 3),
    "two-layer-1M-f64-classical": (_variant(inputs.two_layer_dam_break, "classical"), "f64", 200, 0),
    "two-layer-1M-f64-recompute": (_variant(inputs.two_layer_dam_break), "f64", 200, 3),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_fullsize_variant_parity(name):
    make, prec, nsteps, path = VARIANTS[name]
    w = make()
    say(f"[full variant parity] {name} cells={w.ncells} steps={nsteps} path={path}")
    got, dts, t = gpu_run(w, nsteps=nsteps, path=path, precision=prec)
    say("    gpu done; oracle running")
    if w.nlayers == 2:  # the recomputed-edge run shares the IR-Roe reference of the parity test
        ref, rdts = oracle_reference_cached(("two-layer-1M", w.scheme, nsteps, prec), w, nsteps, prec, chunk=CHUNK)
    else:
        ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    errs = field_errors(got, ref, w.g)
    say(f"    field errors {['%.2e' % e for e in errs]}")
    assert max(errs) <= (FP64_TOL if prec == "f64" else FP32_TOL), errs
    dtol = 1e-12 if prec == "f64" else 1e-5
    derr = np.abs(dts - rdts).max() / rdts.max()
    say(f"    dt error {derr:.2e}")
    assert derr <= dtol
