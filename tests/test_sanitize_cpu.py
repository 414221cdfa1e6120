"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host-side mesh preprocessing (edge derivation, Morton order,
the per-block data of the fused triangle kernels with its 16-bit local ids
and slot codes, Cartesian edge lists) and the oracle's time loops are built
with -fsanitize=address,undefined by g++/gcc and run on the meshes the GPU
tests use: shuffled, ragged and degenerate triangle meshes, one and two
layers, and small grids with walls and periodic sides.  Any out-of-bounds
access, leak or undefined behaviour ends the run with a report.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _have(tool):
    return shutil.which(tool) is not None


pytestmark = pytest.mark.skipif(not (_have("g++") and _have("gcc")), reason="g++/gcc not available")


@pytest.fixture(scope="module")
def harnesses(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    mesh = str(d / "mesh_harness")
    orc = str(d / "oracle_harness")
    r = subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I" + os.path.join(ROOT, "include"),
                        os.path.join(HERE, "sanitize", "mesh_harness.cpp"),
                        os.path.join(ROOT, "finite_volume_shallow_amd", "csrc", "mesh_host.cpp"), "-o", mesh],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run(["gcc", "-std=c11", "-D_GNU_SOURCE", *SAN, "-ffp-contract=off", "-fopenmp",
                        os.path.join(ROOT, "oracle", "swe_oracle.c"), os.path.join(HERE, "sanitize", "oracle_harness.c"),
                        "-o", orc, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return mesh, orc, d


def _shuffled(nq, seed=77):
    w = inputs.circular_dam_break(nq=nq)
    order = np.random.default_rng(seed).permutation(w.ncells)
    w.tri = np.ascontiguousarray(w.tri[order])
    w.z = w.z[order]
    w.state = [a[order] for a in w.state]
    return w


def _tiny(n):
    xy = np.array([[0, 0], [1, 0], [1, 1], [0, 1]], dtype=float)
    tri = np.array([[0, 1, 2], [0, 2, 3]][:n], dtype=np.int32)
    return inputs.Workload(name="tiny", kind="tri", nlayers=1, ntracers=1, precision="f64", g=9.81, r=0.0,
                           cfl=0.9, nsteps=5, z=np.array([0.0, 0.1][:n]),
                           state=[np.array([1.0, 1.3][:n]), np.array([0.2, -0.1][:n]),
                                  np.array([0.1, 0.0][:n]), np.array([0.5, 0.0][:n])],
                           node_xy=xy, tri=tri)


TRI = {
    "tri-36": lambda: inputs.circular_dam_break(nq=36),
    "tri-ragged-19": lambda: inputs.circular_dam_break(nq=19),
    "tri-shuffled-30": lambda: _shuffled(30),
    "two-layer-13": lambda: inputs.two_layer_dam_break(nq=13),
    "one-triangle": lambda: _tiny(1),
    "two-triangles": lambda: _tiny(2),
}


def _write_mesh(path, w):
    xy = np.ascontiguousarray(w.node_xy, dtype=np.float64)
    tri = np.ascontiguousarray(w.tri, dtype=np.int32)
    with open(path, "wb") as f:
        f.write(struct.pack("<qq", xy.shape[0], tri.shape[0]))
        f.write(xy.tobytes())
        f.write(tri.tobytes())


def _run(exe, path):
    r = subprocess.run([exe, path], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and "ERROR" not in r.stderr and "runtime error" not in r.stderr, \
        (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


@pytest.mark.parametrize("name", list(TRI))
def test_mesh_preprocessing_under_sanitizers(harnesses, name):
    mesh, _, d = harnesses
    path = str(d / f"{name}.mesh")
    _write_mesh(path, TRI[name]())
    assert _run(mesh, path).strip().endswith("ok")


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64).tobytes()


ORACLE = {
    "grid-walls-16x8": lambda: inputs.dam_break(nx=16, ny=8),
    "grid-periodic-2x3": lambda: inputs.smooth_flow(nx=2, ny=3),
    "tri-ragged-19": lambda: inputs.circular_dam_break(nq=19),
    "tri-shuffled-20-classical": lambda: _shuffled(20),
    "two-triangles-fix": lambda: _tiny(2),
    "two-layer-13": lambda: inputs.two_layer_dam_break(nq=13),
    "two-layer-9-classical": lambda: inputs.two_layer_dam_break(nq=9),
}


@pytest.mark.parametrize("name", list(ORACLE))
def test_oracle_under_sanitizers(harnesses, name):
    _, orc, d = harnesses
    w = ORACLE[name]()
    classical = int(name.endswith("classical"))
    fix = int(name.endswith("fix"))
    nsteps = 6
    path = str(d / f"{name}.in")
    with open(path, "wb") as f:
        if w.kind == "cart":
            per_y = int(name.startswith("grid-periodic"))
            f.write(struct.pack("<qqqq", 0, nsteps, classical, fix))
            f.write(struct.pack("<qqqq", w.nx, w.ny, int(w.bc_x == "periodic"), per_y))
            f.write(struct.pack("<dd", w.dx, w.dy))
            hc = w.state[3] if w.ntracers else np.zeros(w.ncells)
            for a in (w.z, w.state[0], w.state[1], w.state[2], hc):
                f.write(_f64(a))
        elif w.nlayers == 1:
            f.write(struct.pack("<qqqq", 1, nsteps, classical, fix))
            f.write(struct.pack("<qqq", w.node_xy.shape[0], w.ncells, w.ntracers))
            f.write(_f64(w.node_xy))
            f.write(np.ascontiguousarray(w.tri, dtype=np.int32).tobytes())
            for a in [w.z] + list(w.state):
                f.write(_f64(a))
        else:
            f.write(struct.pack("<qqqq", 2, nsteps, classical, 0))
            f.write(struct.pack("<qq", w.node_xy.shape[0], w.ncells))
            f.write(_f64(w.node_xy))
            f.write(np.ascontiguousarray(w.tri, dtype=np.int32).tobytes())
            for a in [w.z] + list(w.state):
                f.write(_f64(a))
    out = _run(orc, path)
    assert out.startswith("status 0 "), out
    assert float(out.split()[3]) > 0.0
