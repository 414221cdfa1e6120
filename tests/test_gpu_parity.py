"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case runs the same seeded inputs through both and compares every cell
of every conserved field (max relative error per field, normalised by the
field's maximum), the dt of every step and the elapsed time.  fp64 runs must
agree within 1e-10, fp32 runs within 1e-4 after 100 steps.  Sizes are small
enough for the oracle to finish in seconds while spanning many thread blocks
and ragged tails.
"""
import numpy as np
import pytest

import inputs
from helpers import (FP32_TOL, FP64_TOL, field_errors, fsum, gpu_run,
                     oracle_reference, say, tri_areas)

pytestmark = pytest.mark.gpu

PATHS = {"auto": 0, "edge": 1}

def _shuffled_tri(nq, seed=77):
    """the circular dam break with its cells listed in a random order (not Morton)."""
    w = inputs.circular_dam_break(nq=nq)
    order = np.random.default_rng(seed).permutation(w.ncells)
    w.tri = np.ascontiguousarray(w.tri[order])
    w.z = w.z[order]
    w.state = [a[order] for a in w.state]
    return w


def _periodic_xy(nx, ny):
    """the 4096^2-style flow on a small grid, periodic in both directions"""
    w = inputs.smooth_flow(nx=nx, ny=ny)
    w.bc_y = "periodic"
    w.precision = "f64"
    return w


CASES = {
    # name: (workload factory, steps, precision)
    "dam-break-64x64": (lambda: inputs.dam_break(), 100, "f64"),
    "hump-96-f64": (lambda: inputs.gaussian_hump(n=96), 300, "f64"),
    "hump-96-f32": (lambda: inputs.gaussian_hump(n=96), 100, "f32"),
    "flow-160x96-f32": (lambda: inputs.smooth_flow(nx=160, ny=96), 100, "f32"),
    "flow-160x96-f64": (lambda: inputs.smooth_flow(nx=160, ny=96), 150, "f64"),
    "flow-ragged-67x33-f64": (lambda: inputs.smooth_flow(nx=67, ny=33), 80, "f64"),
    "dam-break-ragged-131x5": (lambda: inputs.dam_break(nx=131, ny=5), 60, "f64"),
    "tri-36": (lambda: inputs.circular_dam_break(nq=36), 120, "f64"),
    "tri-ragged-19": (lambda: inputs.circular_dam_break(nq=19), 25, "f64"),
    "two-layer-30": (lambda: inputs.two_layer_dam_break(nq=30), 200, "f64"),
    "two-layer-13": (lambda: inputs.two_layer_dam_break(nq=13), 100, "f64"),
    "two-layer-30-f32": (lambda: inputs.two_layer_dam_break(nq=30), 100, "f32"),
    "tri-shuffled-30": (lambda: _shuffled_tri(30), 60, "f64"),
    "tri-40-f32": (lambda: inputs.circular_dam_break(nq=40), 100, "f32"),
    "flow-periodic-xy-67x40-f64": (lambda: _periodic_xy(67, 40), 60, "f64"),
    "flow-periodic-xy-8x5-f64": (lambda: _periodic_xy(8, 5), 40, "f64"),
}


# Cartesian tilings the size heuristic picks only on large grids, forced on
# small ones: (rows per tile, alternate march direction)
TILINGS = {
    "dam-break-64x64": [(8, 1), (12, 1)],
    "hump-96-f64": [(8, 1), (5, 1)],
    "flow-160x96-f32": [(12, 1), (8, 0)],
    "flow-ragged-67x33-f64": [(4, 1), (12, 1)],
    "dam-break-ragged-131x5": [(4, 1)],
    "flow-periodic-xy-67x40-f64": [(4, 1), (8, 1), (12, 1)],
    # asks for more rows per tile than the periodic grid has: limited to ny - 1
    "flow-periodic-xy-8x5-f64": [(12, 1), (12, 0)],
}


@pytest.mark.parametrize("tiling", [f"{n}@ty{t}alt{a}" for n, v in TILINGS.items() for t, a in v])
def test_parity_cart_tilings(tiling, monkeypatch):
    name, rest = tiling.split("@")
    ty, alt = rest[2:].split("alt")
    monkeypatch.setenv("SWE_CART_TY", ty)
    monkeypatch.setenv("SWE_CART_ALT", alt)
    make, nsteps, prec = CASES[name]
    w = make()
    say(f"[tiling] {name} rows/tile={ty} alternate={alt} steps={nsteps} prec={prec}")
    got, dts, t = gpu_run(w, nsteps=nsteps, precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    errs = field_errors(got, ref, w.g)
    assert max(errs) <= tol, errs
    dtol = 1e-12 if prec == "f64" else 1e-5
    assert np.abs(dts - rdts).max() <= dtol * rdts.max()


# Streaming mode (non-temporal state loads, tile order reversed every other
# step) switches on by itself only where the grid's two state copies and bed
# exceed the last-level cache; here it is forced on small grids.  Tile order
# does not enter the arithmetic and the dt minimum is exact, so the result
# must equal the default run bit for bit, which also shows that the reversed
# order reaches every tile; and it must match the oracle.
STREAMING = {
    "flow-160x96-f32": lambda: CASES["flow-160x96-f32"][0](),
    "flow-ragged-67x33-f64": lambda: CASES["flow-ragged-67x33-f64"][0](),
    "dam-break-ragged-131x5": lambda: CASES["dam-break-ragged-131x5"][0](),
    "flow-periodic-xy-67x40-f64": lambda: CASES["flow-periodic-xy-67x40-f64"][0](),
    "hump-96-f64": lambda: CASES["hump-96-f64"][0](),
    "classical-flow-160x96-f32": lambda: _classical(CASES["flow-160x96-f32"][0]),
    "hh-dam-break-131x5-f32": lambda: HH["hh-dam-break-131x5-f32"][0](),
    "hh-classical-dam-break-200x6-f64": lambda: HH["hh-classical-dam-break-200x6-f64"][0](),
}
STREAM_STEPS = {"hh-dam-break-131x5-f32": (100, "f32"), "hh-classical-dam-break-200x6-f64": (150, "f64"),
                "classical-flow-160x96-f32": (100, "f32")}


def _stream_case(name):
    if name in STREAM_STEPS:
        return STREAMING[name](), *STREAM_STEPS[name]
    _, nsteps, prec = CASES[name]
    return STREAMING[name](), nsteps, prec


STREAM_RUNS = [f"{n}@default" for n in STREAMING] + [
    f"{n}@{v}" for n in ("flow-160x96-f32", "flow-periodic-xy-67x40-f64") for v in ("recompute", "ty8alt1")]


@pytest.mark.parametrize("run", STREAM_RUNS)
def test_parity_cart_streaming(run, monkeypatch):
    name, variant = run.split("@")
    if variant == "ty8alt1":
        monkeypatch.setenv("SWE_CART_TY", "8")
        monkeypatch.setenv("SWE_CART_ALT", "1")
    path = 3 if variant == "recompute" else 0
    w, nsteps, prec = _stream_case(name)
    say(f"[streaming] {name} {variant} steps={nsteps} prec={prec}")
    monkeypatch.setenv("SWE_CART_STREAM", "0")
    base, bdts, bt = gpu_run(w, nsteps=nsteps, path=path, precision=prec)
    monkeypatch.setenv("SWE_CART_STREAM", "1")
    got, dts, t = gpu_run(w, nsteps=nsteps, path=path, precision=prec)
    assert np.array_equal(dts, bdts) and t == bt
    for a, b in zip(got, base):
        assert np.array_equal(a, b)
    if variant == "default":
        ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
        tol = FP64_TOL if prec == "f64" else FP32_TOL
        errs = field_errors(got, ref, w.g)
        assert max(errs) <= tol, errs
        dtol = 1e-12 if prec == "f64" else 1e-5
        assert np.abs(dts - rdts).max() <= dtol * rdts.max()


def test_streaming_across_batches(monkeypatch):
    """The order alternates with the state buffer a step reads, so a run
    split into batches of odd lengths equals one batch bit for bit."""
    import finite_volume_shallow_amd as swe
    w = inputs.smooth_flow(nx=160, ny=96)
    say("[streaming] 7 + 6 + 5 steps == 18 steps")
    monkeypatch.setenv("SWE_CART_STREAM", "0")
    a, da, _ = gpu_run(w, nsteps=18)
    monkeypatch.setenv("SWE_CART_STREAM", "1")
    desc, keep = swe.desc_from_workload(w)
    ctx = swe.swe_create_mesh(desc)
    try:
        swe.swe_set_state(ctx, w.z, w.state)
        for n in (7, 6, 5):
            swe.swe_step(ctx, n, w.cfl)
        b = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    del keep
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# One-layer triangle meshes run the software-pipelined persistent kernel by
# default; these force the one-workgroup-per-block kernel (and its larger
# blocks) on them, and the pipelined kernel with smaller blocks and small
# persistent grids: with one or three workgroups per XCD band most blocks
# of these meshes are taken from the band's counter (positions from twice
# the workgroups per band on), which the default grid reaches only on
# meshes of several hundred thousand cells.
TRI_KERNELS = {"per-block-288": {"SWE_TRI_PIPE": "0", "SWE_TRI_B": "288"},
               "per-block-128": {"SWE_TRI_PIPE": "0", "SWE_TRI_B": "128"},
               "pipelined-128": {"SWE_TRI_B": "128"},
               "pipelined-64-1wg": {"SWE_TRI_B": "64", "SWE_TRI_WGS": "8"},
               "pipelined-64-3wg": {"SWE_TRI_B": "64", "SWE_TRI_WGS": "24"}}


@pytest.mark.parametrize("kernel", list(TRI_KERNELS))
@pytest.mark.parametrize("name", ["tri-36", "tri-ragged-19", "tri-shuffled-30", "tri-40-f32"])
def test_parity_tri_kernels(name, kernel, monkeypatch):
    for k, v in TRI_KERNELS[kernel].items():
        monkeypatch.setenv(k, v)
    make, nsteps, prec = CASES[name]
    w = make()
    say(f"[tri kernel] {name} {kernel} steps={nsteps} prec={prec}")
    got, dts, t = gpu_run(w, nsteps=nsteps, precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    errs = field_errors(got, ref, w.g)
    assert max(errs) <= tol, errs
    dtol = 1e-12 if prec == "f64" else 1e-5
    assert np.abs(dts - rdts).max() <= dtol * rdts.max()


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", list(CASES))
def test_parity(name, path):
    make, nsteps, prec = CASES[name]
    w = make()
    say(f"[parity] {name} path={path} steps={nsteps} prec={prec} cells={w.ncells}")
    got, dts, t = gpu_run(w, nsteps=nsteps, path=PATHS[path], precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    errs = field_errors(got, ref, w.g)
    say(f"    field errors {['%.2e' % e for e in errs]}")
    assert max(errs) <= tol, errs
    assert dts.shape == rdts.shape
    dtol = 1e-12 if prec == "f64" else 1e-5
    assert np.abs(dts - rdts).max() <= dtol * rdts.max()
    assert abs(t - rdts.sum()) <= dtol * rdts.sum()


def _tri_pollutant(nq, seed=91):
    """the triangle dam break with a pollutant: concentration a seeded
    smooth field in [0.2, 1] (no triangle workload carries one)"""
    w = inputs.circular_dam_break(nq=nq)
    rng = np.random.default_rng(seed)
    xy = w.node_xy[w.tri].mean(axis=1)
    kx, ky, ph = rng.uniform(1.0, 4.0), rng.uniform(1.0, 4.0), rng.uniform(0, 2 * np.pi)
    conc = 0.6 + 0.4 * np.sin(2 * np.pi * (kx * xy[:, 0] + ky * xy[:, 1]) / 1000.0 + ph)
    w.ntracers = 1
    w.state = w.state + [w.state[0] * conc]
    return w


# The classical Roe flux (contact waves of the Roe velocity for the
# transverse momentum and the pollutant) on every case, both paths.
CLASSICAL = dict(CASES)
CLASSICAL["tri-pollutant-23"] = (lambda: _tri_pollutant(23), 80, "f64")
CLASSICAL["tri-pollutant-33-f32"] = (lambda: _tri_pollutant(33), 80, "f32")


def _classical(make):
    w = make()
    w.scheme = "classical"
    return w


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", list(CLASSICAL))
def test_parity_classical(name, path):
    make, nsteps, prec = CLASSICAL[name]
    w = _classical(make)
    say(f"[classical] {name} path={path} steps={nsteps} prec={prec} cells={w.ncells}")
    got, dts, t = gpu_run(w, nsteps=nsteps, path=PATHS[path], precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    errs = field_errors(got, ref, w.g)
    say(f"    field errors {['%.2e' % e for e in errs]}")
    assert max(errs) <= tol, errs
    dtol = 1e-12 if prec == "f64" else 1e-5
    assert np.abs(dts - rdts).max() <= dtol * rdts.max()
    assert abs(t - rdts.sum()) <= dtol * rdts.sum()


@pytest.mark.parametrize("kernel", list(TRI_KERNELS))
@pytest.mark.parametrize("name", ["tri-pollutant-23", "tri-40-f32", "two-layer-13"])
def test_parity_classical_tri_kernels(name, kernel, monkeypatch):
    for k, v in TRI_KERNELS[kernel].items():
        monkeypatch.setenv(k, v)
    make, nsteps, prec = CLASSICAL[name]
    w = _classical(make)
    say(f"[classical tri kernel] {name} {kernel} steps={nsteps} prec={prec}")
    got, dts, t = gpu_run(w, nsteps=nsteps, precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    assert max(field_errors(got, ref, w.g)) <= tol
    dtol = 1e-12 if prec == "f64" else 1e-5
    assert np.abs(dts - rdts).max() <= dtol * rdts.max()


def test_parity_ir_pollutant_triangles():
    # the IR-Roe pollutant on triangle meshes (both paths)
    for path in PATHS:
        w = _tri_pollutant(23)
        say(f"[ir pollutant tri] path={path}")
        got, dts, t = gpu_run(w, nsteps=80, path=PATHS[path])
        ref, rdts = oracle_reference(w, nsteps=80)
        assert max(field_errors(got, ref, w.g)) <= FP64_TOL
        assert np.abs(dts - rdts).max() <= 1e-12 * rdts.max()


def test_classical_and_ir_differ_on_gpu():
    # the two schemes share mass and normal momentum fluxes but not the
    # pollutant's: after a few steps of a sheared flow they must differ
    w = inputs.smooth_flow(nx=64, ny=40)
    w.precision = "f64"
    ir, _, _ = gpu_run(w, nsteps=20)
    cl, _, _ = gpu_run(_classical(lambda: w.copy()), nsteps=20)
    assert np.abs(ir[3] - cl[3]).max() > 1e-8 * np.abs(ir[3]).max()


# The recomputation variants of the fused kernels (every cell evaluates all
# of its edges itself): against the oracle, and against the shared-edge
# kernels (on Cartesian grids in every tiling and march direction).  A
# recomputed edge has the same inputs as the shared one, but the compiler
# may contract its multiply-adds differently, so the two agree to rounding:
# in float32 that rounding accumulates over 100 steps to the size of the
# float32-vs-float64 error itself (2.6e-5 on the 96^2 hump), so the bar is
# half of the 1e-4 float32 tolerance.
RC_TOL = {"f64": 1e-12, "f32": 5e-5}


@pytest.mark.parametrize("name", list(CASES))
def test_parity_recompute(name):
    make, nsteps, prec = CASES[name]
    w = make()
    say(f"[recompute] {name} steps={nsteps} prec={prec}")
    got, dts, t = gpu_run(w, nsteps=nsteps, path=3, precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    assert max(field_errors(got, ref, w.g)) <= tol
    dtol = 1e-12 if prec == "f64" else 1e-5
    assert np.abs(dts - rdts).max() <= dtol * rdts.max()
    shared, sdts, _ = gpu_run(w, nsteps=nsteps, path=2, precision=prec)
    errs = field_errors(got, shared, w.g)
    say(f"    recompute vs shared {['%.2e' % e for e in errs]}")
    assert max(errs) <= RC_TOL[prec], errs
    assert np.abs(dts - sdts).max() <= RC_TOL[prec] * sdts.max()


@pytest.mark.parametrize("tiling", [f"{n}@ty{t}alt{a}" for n, v in TILINGS.items() for t, a in v])
def test_recompute_in_every_tiling(tiling, monkeypatch):
    name, rest = tiling.split("@")
    ty, alt = rest[2:].split("alt")
    monkeypatch.setenv("SWE_CART_TY", ty)
    monkeypatch.setenv("SWE_CART_ALT", alt)
    make, nsteps, prec = CASES[name]
    w = make()
    say(f"[recompute tiling] {name} rows/tile={ty} alternate={alt}")
    a, da, _ = gpu_run(w, nsteps=min(nsteps, 40), path=3, precision=prec)
    b, db, _ = gpu_run(w, nsteps=min(nsteps, 40), path=2, precision=prec)
    errs = field_errors(a, b, w.g)
    assert max(errs) <= RC_TOL[prec], errs
    assert np.abs(da - db).max() <= RC_TOL[prec] * db.max()


# The Harten-Hyman entropy fix: transonic dam breaks (the rarefaction
# straddles the dam, so the fix acts every step) on a Cartesian strip and a
# triangle mesh, and ordinary workloads with the fix switched on.
def _transonic_cart(nx, ny):
    w = inputs.dam_break(nx=nx, ny=ny)
    x = (np.arange(nx) + 0.5) * w.dx
    left = np.tile(x < nx * w.dx / 2, ny)
    h = np.where(left, 1.0, 0.05)
    w.state = [h, np.zeros_like(h), np.zeros_like(h), h * np.where(left, 1.0, 0.2)]
    w.entropy_fix = 1
    return w


def _transonic_tri(nq):
    w = inputs.circular_dam_break(nq=nq)
    w.z = np.zeros_like(w.z)
    w.state[0] = np.where(w.state[0] > 2.0, 3.0, 0.12)
    w.entropy_fix = 1
    return w


def _with_fix(make):
    def f():
        w = make()
        w.entropy_fix = 1
        return w
    return f


HH = {
    "hh-dam-break-200x6-f64": (lambda: _transonic_cart(200, 6), 150, "f64"),
    "hh-dam-break-131x5-f32": (lambda: _transonic_cart(131, 5), 100, "f32"),
    "hh-tri-circular-24-f64": (lambda: _transonic_tri(24), 80, "f64"),
    "hh-tri-circular-30-f32": (lambda: _transonic_tri(30), 60, "f32"),
    "hh-flow-160x96-f32": (_with_fix(CASES["flow-160x96-f32"][0]), 100, "f32"),
    "hh-tri-ragged-19": (_with_fix(CASES["tri-ragged-19"][0]), 25, "f64"),
    # the classical flux with the fix
    "hh-classical-dam-break-200x6-f64": (lambda: _classical(lambda: _transonic_cart(200, 6)), 150, "f64"),
    "hh-classical-tri-circular-24-f64": (lambda: _classical(lambda: _transonic_tri(24)), 80, "f64"),
    "hh-classical-dam-break-131x5-f32": (lambda: _classical(lambda: _transonic_cart(131, 5)), 100, "f32"),
}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", list(HH))
def test_parity_entropy_fix(name, path):
    make, nsteps, prec = HH[name]
    w = make()
    say(f"[entropy fix] {name} path={path} steps={nsteps} prec={prec}")
    got, dts, t = gpu_run(w, nsteps=nsteps, path=PATHS[path], precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    errs = field_errors(got, ref, w.g)
    say(f"    field errors {['%.2e' % e for e in errs]}")
    assert max(errs) <= tol, errs
    dtol = 1e-12 if prec == "f64" else 1e-5
    assert np.abs(dts - rdts).max() <= dtol * rdts.max()


@pytest.mark.parametrize("variant", ["ty4alt1", "ty12alt1", "per-block-128", "per-block-288"])
def test_parity_entropy_fix_kernel_variants(variant, monkeypatch):
    if variant.startswith("ty"):
        ty, alt = variant[2:].split("alt")
        monkeypatch.setenv("SWE_CART_TY", ty)
        monkeypatch.setenv("SWE_CART_ALT", alt)
        make, nsteps, prec = HH["hh-dam-break-200x6-f64"]
    else:
        for k, v in TRI_KERNELS[variant].items():
            monkeypatch.setenv(k, v)
        make, nsteps, prec = HH["hh-tri-circular-24-f64"]
    w = make()
    say(f"[entropy fix variant] {variant}")
    got, dts, _ = gpu_run(w, nsteps=nsteps, precision=prec)
    ref, rdts = oracle_reference(w, nsteps=nsteps, precision=prec)
    assert max(field_errors(got, ref, w.g)) <= FP64_TOL
    assert np.abs(dts - rdts).max() <= 1e-12 * rdts.max()


def test_entropy_fix_acts_on_gpu():
    for make in (lambda: _transonic_cart(200, 6), lambda: _transonic_tri(24)):
        w = make()
        fixed, _, _ = gpu_run(w, nsteps=60)
        w.entropy_fix = 0
        plain, _, _ = gpu_run(w, nsteps=60)
        assert np.abs(fixed[0] - plain[0]).max() > 1e-3


def test_dam_break_symmetry_on_gpu():
    w = inputs.dam_break()
    say("[sym] dam_break rows identical, qy == 0")
    got, _, _ = gpu_run(w)
    assert np.abs(got[2]).max() <= 1e-14
    for a in got:
        g2 = a.reshape(64, 64)
        assert np.abs(g2 - g2[0]).max() <= 1e-14 * max(np.abs(g2).max(), 1.0)


def test_conservation_on_gpu():
    say("[cons] gaussian_hump 96^2 and two_layer_dam_break 30 conservation")
    w = inputs.gaussian_hump(n=96)
    got, _, _ = gpu_run(w, nsteps=500)
    area = w.dx * w.dy
    for v in (0, 3):
        assert abs(fsum(got[v]) - fsum(w.state[v])) * area <= 1e-12 * fsum(w.state[v]) * area
    w = inputs.two_layer_dam_break(nq=30)
    got, _, _ = gpu_run(w, nsteps=200)
    ar = tri_areas(w)
    for v in (0, 3):
        m0 = fsum(w.state[v] * ar)
        assert abs(fsum(got[v] * ar) - m0) <= 1e-12 * m0


def test_lake_at_rest_on_gpu():
    say("[rest] lake at rest, Cartesian fp64 and fp32, triangles")
    w = inputs.gaussian_hump(n=96, hump=False, blob=False)
    got, _, _ = gpu_run(w, nsteps=500)
    assert np.abs(got[1] / got[0]).max() <= 1e-12
    assert np.abs(got[0] + w.z - 5.0).max() <= 1e-12
    got, _, _ = gpu_run(w, nsteps=200, precision="f32")
    z32 = w.z.astype(np.float32).astype(np.float64)
    assert np.abs(got[1] / got[0]).max() <= 1e-5
    assert np.abs(got[0] + z32 - 5.0).max() <= 1e-5
    w = inputs.circular_dam_break(nq=24, still=True)
    got, _, _ = gpu_run(w, nsteps=200)
    assert np.abs(got[1] / got[0]).max() <= 1e-12
    assert np.abs(got[0] + w.z - 5.0).max() <= 1e-12


def test_determinism_and_resume():
    import finite_volume_shallow_amd as swe
    w = inputs.circular_dam_break(nq=30)
    say("[det] two runs bitwise equal; 2n steps == n + get/set + n")
    a, da, _ = gpu_run(w, nsteps=40)
    b, db, _ = gpu_run(w, nsteps=40)
    assert (da == db).all()
    for x, y in zip(a, b):
        assert (x == y).all()
    desc, keep = swe.desc_from_workload(w)
    ctx = swe.swe_create_mesh(desc)
    try:
        swe.swe_set_state(ctx, w.z, w.state)
        swe.swe_step(ctx, 20, w.cfl)
        mid = swe.swe_get_state(ctx)
        swe.swe_set_state(ctx, w.z, mid)
        swe.swe_step(ctx, 20, w.cfl)
        c = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    for x, y in zip(a, c):
        assert (x == y).all()


def test_device_state_roundtrip_and_stream():
    import torch
    import finite_volume_shallow_amd as swe
    say("[dev] device set/get on a torch stream")
    w = inputs.smooth_flow(nx=64, ny=40)
    s = torch.cuda.Stream()
    desc, keep = swe.desc_from_workload(w, stream=s, precision="f32")
    ctx = swe.swe_create_mesh(desc)
    try:
        dev = [torch.tensor(a, dtype=torch.float32, device="cuda") for a in w.state]
        z = torch.tensor(w.z, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        swe.swe_set_state_device(ctx, z, dev)
        swe.swe_step(ctx, 30, w.cfl)
        outs = [torch.empty_like(d) for d in dev]
        swe.swe_get_state_device(ctx, outs)
        s.synchronize()
        host = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    for o, h in zip(outs, host):
        assert (o.cpu().double().numpy() == h).all()
    got, _, _ = gpu_run(w, nsteps=30, precision="f32")
    for o, g in zip(host, got):
        assert (o == g).all()


def test_two_contexts_interleaved():
    """Two live contexts, each on its own stream, stepped in alternating
    batches: each matches its own oracle run (contexts share nothing)."""
    import torch
    import finite_volume_shallow_amd as swe
    say("[ctx] a Cartesian and a triangle context interleaved on two streams")
    wa = inputs.dam_break(nx=40, ny=24)
    wb = inputs.circular_dam_break(nq=14)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    da, ka = swe.desc_from_workload(wa, stream=sa)
    db, kb = swe.desc_from_workload(wb, stream=sb)
    ca = swe.swe_create_mesh(da)
    try:
        cb = swe.swe_create_mesh(db)
        try:
            swe.swe_set_state(ca, wa.z, wa.state)
            swe.swe_set_state(cb, wb.z, wb.state)
            ta = tb = 0.0
            for _ in range(3):
                ta += swe.swe_step(ca, 10, wa.cfl)[0]
                tb += swe.swe_step(cb, 10, wb.cfl)[0]
            got_a, got_b = swe.swe_get_state(ca), swe.swe_get_state(cb)
        finally:
            swe.swe_destroy(cb)
    finally:
        swe.swe_destroy(ca)
    for w, got, t in ((wa, got_a, ta), (wb, got_b, tb)):
        ref, rdts = oracle_reference(w, nsteps=30)
        assert max(field_errors(got, ref, w.g)) <= FP64_TOL
        assert abs(t - rdts.sum()) <= 1e-12 * rdts.sum()


def test_device_state_roundtrip_triangles():
    import torch
    import finite_volume_shallow_amd as swe
    say("[dev] device set/get on a permuted triangle mesh")
    w = _shuffled_tri(24)
    desc, keep = swe.desc_from_workload(w)
    ctx = swe.swe_create_mesh(desc)
    try:
        dev = [torch.tensor(a, dtype=torch.float64, device="cuda") for a in w.state]
        z = torch.tensor(w.z, dtype=torch.float64, device="cuda")
        torch.cuda.synchronize()
        swe.swe_set_state_device(ctx, z, dev)
        swe.swe_step(ctx, 20, w.cfl)
        outs = [torch.empty_like(d) for d in dev]
        swe.swe_get_state_device(ctx, outs)
        torch.cuda.synchronize()
        host = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    got, _, _ = gpu_run(w, nsteps=20)
    for o, h, g in zip(outs, host, got):
        assert (o.cpu().numpy() == h).all()
        assert (h == g).all()


def _describe(w, **kw):
    import finite_volume_shallow_amd as swe
    desc, keep = swe.desc_from_workload(w, **kw)
    ctx = swe.swe_create_mesh(desc)
    try:
        return swe.swe_describe(ctx)
    finally:
        swe.swe_destroy(ctx)


def test_describe_names_the_kernel():
    say("[describe] structured, triangles, two layers, edge path")
    d = _describe(inputs.smooth_flow(nx=160, ny=96))
    assert d.startswith("IR-Roe flux, float32") and "structured grid 160 x 96" in d, d
    assert "tiles of 60 columns" in d and "streaming" not in d, d
    d = _describe(_classical(lambda: inputs.circular_dam_break(nq=36)))
    assert d.startswith("classical Roe flux, float64"), d
    assert "one layer: software-pipelined persistent kernel, blocks of 224 cells" in d, d
    d = _describe(inputs.two_layer_dam_break(nq=30))
    assert "two layers: one workgroup per block" in d, d
    d = _describe(inputs.dam_break(), path=PATHS["edge"])
    assert "edge-list path" in d, d


def test_pipelined_schedules_agree_bit_for_bit(monkeypatch):
    """The same blocks run by one, three or as many persistent workgroups per
    XCD band as fit (block order and the band counters differ) give the same
    bits: no block's arithmetic depends on which workgroup runs it, and the
    dt minimum is exact."""
    w = inputs.circular_dam_break(nq=60)
    monkeypatch.setenv("SWE_TRI_B", "64")
    runs = []
    for wgs in ("8", "24", None):
        if wgs is None:
            monkeypatch.delenv("SWE_TRI_WGS", raising=False)
        else:
            monkeypatch.setenv("SWE_TRI_WGS", wgs)
        say(f"[schedules] {_describe(w)}; workgroups {wgs or 'as many as fit'}")
        runs.append(gpu_run(w, nsteps=30))
    (a, da, ta) = runs[0]
    for b, db, tb in runs[1:]:
        assert np.array_equal(da, db) and ta == tb
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    ref, rdts = oracle_reference(w, nsteps=30)
    assert max(field_errors(a, ref, w.g)) <= FP64_TOL
    assert np.abs(da - rdts).max() <= 1e-12 * rdts.max()


def test_pipelined_kernel_mid_size_mesh():
    """405,000 triangles: 1,809 blocks, so each XCD band has more than twice
    the default persistent workgroups per band and the later blocks come from
    the band counters.  Two batches, so the counters are reset between them."""
    import finite_volume_shallow_amd as swe
    w = inputs.circular_dam_break(nq=450)
    say(f"[mid] {_describe(w)}")
    ref, rdts = oracle_reference(w, nsteps=12)
    desc, keep = swe.desc_from_workload(w)
    ctx = swe.swe_create_mesh(desc)
    try:
        swe.swe_set_state(ctx, w.z, w.state)
        swe.swe_step(ctx, 5, w.cfl)
        d1 = swe.swe_get_dt_history(ctx)
        swe.swe_step(ctx, 7, w.cfl)
        d2 = swe.swe_get_dt_history(ctx)
        got = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    del keep
    errs = field_errors(got, ref, w.g)
    assert max(errs) <= FP64_TOL, errs
    dts = np.concatenate([d1, d2])
    assert np.abs(dts - rdts).max() <= 1e-12 * rdts.max()
    again, _, _ = gpu_run(w, nsteps=12)
    for a, b in zip(got, again):
        assert np.array_equal(a, b)


def test_pipelined_kernel_shrinks_its_blocks():
    """On the jittered 1M-triangle mesh a few blocks of 224 cells have more
    than 512 local edges; the pipelined kernel is kept, at 216 cells."""
    w = inputs.circular_dam_break(nq=707)
    d = _describe(w)
    say(f"[shrink] {d}")
    assert "software-pipelined persistent kernel, blocks of 216 cells" in d, d
    got, dts, _ = gpu_run(w, nsteps=6)
    ref, rdts = oracle_reference(w, nsteps=6)
    errs = field_errors(got, ref, w.g)
    assert max(errs) <= FP64_TOL, errs
    assert np.abs(dts - rdts).max() <= 1e-12 * rdts.max()


def test_error_paths():
    import finite_volume_shallow_amd as swe
    say("[err] depth, non-hyperbolic, bad arguments, zero steps")
    w = inputs.dam_break(nx=16, ny=8)
    w.state[0][17] = -0.5
    with pytest.raises(swe.SweError) as e:
        gpu_run(w, nsteps=2)
    assert e.value.status == swe.SWE_E_DEPTH

    # a non-finite pollutant leaves depth and momentum alone (the pollutant
    # does not feed back) but is reported, on both fused paths and the edge path
    for make in (lambda: inputs.dam_break(nx=16, ny=8), lambda: _tri_pollutant(8)):
        for path in (0, 1):
            w = make()
            w.state[3][20] = np.inf
            with pytest.raises(swe.SweError) as e:
                gpu_run(w, nsteps=2, path=path)
            assert e.value.status == swe.SWE_E_NONFINITE

    w = inputs.two_layer_dam_break(nq=6)
    for v in (1, 4):
        w.state[v] = (1.5 if v == 1 else -1.5) * w.state[v - 1]
    with pytest.raises(swe.SweError) as e:
        gpu_run(w, nsteps=1)
    assert e.value.status == swe.SWE_E_NONHYPERBOLIC

    w = inputs.dam_break(nx=8, ny=8)
    desc, keep = swe.desc_from_workload(w)
    ctx = swe.swe_create_mesh(desc)
    try:
        with pytest.raises(swe.SweError) as e:
            swe.swe_step(ctx, 1, 0.9)
        assert e.value.status == swe.SWE_E_NOSTATE
        swe.swe_set_state(ctx, w.z, w.state)
        for bad in ((-1, 0.9), (1, 0.0), (1, 1.5)):
            with pytest.raises(swe.SweError) as e:
                swe.swe_step(ctx, *bad)
            assert e.value.status == swe.SWE_E_INVAL
        assert swe.swe_step(ctx, 0, 0.9) == (0.0, 0.0)
        got = swe.swe_get_state(ctx)
        for a, b in zip(got, w.state):
            assert (a == b).all()
        # the binding checks array counts and lengths before the library
        # would read past a short array
        with pytest.raises(ValueError):
            swe.swe_set_state(ctx, w.z, w.state[:3])
        with pytest.raises(ValueError):
            swe.swe_set_state(ctx, w.z, [a[:-1] for a in w.state])
        with pytest.raises(ValueError):
            swe.swe_set_state(ctx, w.z[:-1], w.state)
        import torch
        dev = [torch.zeros(w.ncells + 1, dtype=torch.float64, device="cuda") for _ in w.state]
        with pytest.raises(ValueError):
            swe.swe_get_state_device(ctx, dev)
    finally:
        swe.swe_destroy(ctx)


@pytest.mark.parametrize("case", ["2x2-walls", "2x3-periodic", "one-triangle", "two-triangles"])
def test_degenerate_meshes(case):
    say(f"[degenerate] {case}")
    if case == "2x2-walls":
        w = inputs.dam_break(nx=2, ny=2)
        w.state[0] = np.array([2.0, 1.0, 1.5, 1.2])
    elif case == "2x3-periodic":
        w = inputs.smooth_flow(nx=2, ny=3)
        w.bc_y = "periodic"
        w.precision = "f64"
    else:
        xy = np.array([[0, 0], [1, 0], [1, 1], [0, 1]], dtype=float)
        tri = np.array([[0, 1, 2]] if case == "one-triangle" else [[0, 1, 2], [0, 2, 3]], dtype=np.int32)
        n = tri.shape[0]
        w = inputs.Workload(name=case, kind="tri", nlayers=1, ntracers=1, precision="f64",
                            g=9.81, r=0.0, cfl=0.9, nsteps=10, z=np.array([0.0, 0.1][:n]),
                            state=[np.array([1.0, 1.3][:n]), np.array([0.2, -0.1][:n]),
                                   np.array([0.1, 0.0][:n]), np.array([0.5, 0.0][:n])],
                            node_xy=xy, tri=tri)
    got, dts, _ = gpu_run(w, nsteps=10, precision="f64")
    ref, rdts = oracle_reference(w, nsteps=10, precision="f64")
    assert max(field_errors(got, ref)) <= FP64_TOL
    assert np.abs(dts - rdts).max() <= 1e-12 * rdts.max()


# Consecutive swe_step calls continue one time stepping: a call with the same
# cfl starts from the dt the previous call's last step computed, so several
# calls equal one call of the summed step count bit for bit.
SPLIT = {"dam-break-64x64": {}, "flow-160x96-f32": {}, "tri-36": {}, "tri-36-per-block": {"SWE_TRI_PIPE": "0"},
         "two-layer-13": {}, "tri-40-f32": {}}


@pytest.mark.parametrize("path", ["auto", "recompute", "edge"])
@pytest.mark.parametrize("name", list(SPLIT))
def test_consecutive_calls_continue_one_stepping(name, path, monkeypatch):
    import finite_volume_shallow_amd as swe
    for k, v in SPLIT[name].items():
        monkeypatch.setenv(k, v)
    make, _, prec = CASES[name.replace("-per-block", "")]
    w = make()
    p = {"auto": swe.SWE_PATH_AUTO, "recompute": swe.SWE_PATH_RECOMPUTE, "edge": swe.SWE_PATH_EDGE}[path]
    say(f"[split calls] {name} path={path}")
    whole, whole_dts, whole_t = gpu_run(w, nsteps=23, path=p, precision=prec)
    desc, keep = swe.desc_from_workload(w, path=p, precision=prec)
    ctx = swe.swe_create_mesh(desc)
    try:
        swe.swe_set_state(ctx, w.z, w.state)
        dts, t = [], 0.0
        for n in (1, 1, 5, 16):
            t += swe.swe_step(ctx, n, w.cfl)[0]
            dts.append(swe.swe_get_dt_history(ctx))
        got = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    assert (np.concatenate(dts) == whole_dts).all()
    for a, b in zip(got, whole):
        assert (a == b).all()
    assert abs(t - whole_t) <= 1e-14 * whole_t


@pytest.mark.parametrize("name", ["dam-break-64x64", "tri-36", "flow-160x96-f32"])
def test_cfl_change_and_new_state_between_calls(name):
    """A call with another cfl, and a call after a new set_state, start by
    computing dt of the state they find: matches the oracle run in the same
    segments."""
    import finite_volume_shallow_amd as swe
    make, _, prec = CASES[name]
    w = make()
    say(f"[cfl change] {name}")
    desc, keep = swe.desc_from_workload(w, precision=prec)
    ctx = swe.swe_create_mesh(desc)
    try:
        swe.swe_set_state(ctx, w.z, w.state)
        swe.swe_step(ctx, 10, 0.9)
        swe.swe_step(ctx, 10, 0.5)
        seg = swe.swe_get_dt_history(ctx)
        got = swe.swe_get_state(ctx)
        # a new state: the next call must not reuse the old dt
        swe.swe_set_state(ctx, w.z, w.state)
        swe.swe_step(ctx, 10, 0.9)
        again = swe.swe_get_state(ctx)
    finally:
        swe.swe_destroy(ctx)
    w1 = w.copy()
    w1.cfl = 0.9
    mid, d1 = oracle_reference(w1, nsteps=10, precision=prec)
    w2 = w.copy(state=[np.asarray(a, dtype=np.float64) for a in mid], precision="f64")
    w2.cfl = 0.5
    ref, d2 = oracle_reference(w2, nsteps=10)
    tol = FP64_TOL if prec == "f64" else FP32_TOL
    assert max(field_errors(got, ref, w.g)) <= tol
    assert np.abs(seg - d2).max() <= (1e-12 if prec == "f64" else 1e-5) * d2.max()
    assert max(field_errors(again, mid, w.g)) <= tol
