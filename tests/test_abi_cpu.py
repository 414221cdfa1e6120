"""C-ABI checks that need no GPU: the library loads, exports every function
include/swe.h declares, and rejects bad descriptions before any device work.
"""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import finite_volume_shallow_amd as swe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "swe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swe_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    declared = _declared()
    assert len(declared) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", swe.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    assert sorted(swe.EXPORTS) == declared


def test_struct_layout_matches_header():
    # offsets follow the C layout of swe_mesh_desc on x86-64
    d = swe.swe_mesh_desc
    assert d.scheme.offset == 24 and d.entropy_fix.offset == 28 and d.g.offset == 32 and d.nx.offset == 48
    assert d.bc_x.offset == 80 and d.nnodes.offset == 88 and d.node_xy.offset == 104
    assert d.hip_stream.offset == 120 and ctypes.sizeof(d) == 128


def test_binding_constants_match_header():
    # every enum value and the ABI version the binding uses is the header's
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "swe.h")).read()
    assert int(re.search(r"#define SWE_ABI_VERSION (\d+)", hdr).group(1)) == swe.SWE_ABI_VERSION
    consts = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(SWE_[A-Z0-9_]+) = (-?\d+)", hdr)}
    for name in ["SWE_MESH_CART", "SWE_MESH_TRI", "SWE_F64", "SWE_F32", "SWE_BC_WALL", "SWE_BC_PERIODIC",
                 "SWE_PATH_AUTO", "SWE_PATH_EDGE", "SWE_PATH_FUSED", "SWE_PATH_RECOMPUTE",
                 "SWE_SCHEME_IR_ROE", "SWE_SCHEME_ROE", "SWE_ENTROPY_FIX_NONE", "SWE_ENTROPY_FIX_HH"]:
        assert consts[name] == getattr(swe, name), name


def test_strerror_covers_all_codes():
    for code in range(0, -8, -1):
        assert swe.swe_strerror(code) != "unknown status"
    assert swe.swe_strerror(-99) == "unknown status"


def _cart(**kw):
    args = dict(kind="cart", nx=8, ny=8, dx=1.0, dy=1.0)
    args.update(kw)
    return swe.mesh_desc(**args)


@pytest.mark.parametrize("kw, msg", [
    (dict(nx=1), "nx and ny"),
    (dict(dx=0.0), "dx and dy"),
    (dict(g=-1.0), "g must"),
    (dict(nlayers=2, r=0.5), "two layers"),
    (dict(nlayers=3), "nlayers"),
    (dict(ntracers=2), "ntracers"),
    (dict(precision=7), None),
])
def test_create_rejects_bad_cartesian(kw, msg):
    kw = dict(kw)
    code = kw.pop("precision", None)  # an out-of-enum code, set past the binding's check
    d, keep = _cart(**kw)
    if code is not None:
        d.precision = code
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL
    if msg:
        assert msg in str(e.value)


def test_create_rejects_bad_abi_version():
    d, keep = _cart()
    d.abi_version = 99
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL


def _square_mesh():
    xy = np.array([[0, 0], [1, 0], [1, 1], [0, 1]], dtype=float)
    tri = np.array([[0, 1, 2], [0, 2, 3]], dtype=np.int32)
    return xy, tri


def test_recompute_path_is_ir_roe_only():
    xy, tri = _square_mesh()
    d, keep = swe.mesh_desc(kind="tri", node_xy=xy, tri=tri, path=swe.SWE_PATH_RECOMPUTE, scheme="classical")
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL and "recomputation" in str(e.value)
    d, keep = _cart()
    d.path = swe.SWE_PATH_RECOMPUTE
    d.scheme = swe.SWE_SCHEME_ROE
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL
    d.path = 4
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL


def test_entropy_fix_is_one_layer_only():
    for kw in (dict(path=swe.SWE_PATH_RECOMPUTE),):
        d, keep = swe.mesh_desc(kind="cart", nx=8, ny=8, dx=1.0, dy=1.0, entropy_fix=1, **kw)
        with pytest.raises(swe.SweError) as e:
            swe.swe_create_mesh(d)
        assert e.value.status == swe.SWE_E_INVAL and "entropy" in str(e.value)
    xy, tri = _square_mesh()
    d, keep = swe.mesh_desc(kind="tri", node_xy=xy, tri=tri, nlayers=2, r=0.9, entropy_fix=1)
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL
    d, keep = _cart()
    d.entropy_fix = 3
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL


def test_create_rejects_bad_scheme():
    d, keep = _cart()
    d.scheme = 5
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL and "scheme" in str(e.value)
    with pytest.raises(ValueError):
        swe.mesh_desc(kind="cart", nx=4, ny=4, dx=1.0, dy=1.0, scheme="hllc")


@pytest.mark.parametrize("field,value", [("kind", "hex"), ("precision", "f16"), ("bc_x", "periodc"),
                                         ("bc_y", "open")])
def test_mesh_desc_rejects_unknown_names(field, value):
    kw = dict(kind="cart", nx=4, ny=4, dx=1.0, dy=1.0)
    kw[field] = value
    with pytest.raises(ValueError, match=field):
        swe.mesh_desc(**kw)


@pytest.mark.parametrize("case", ["clockwise", "node-range", "triple-edge", "two-layer-tracer", "bad-r"])
def test_create_rejects_bad_triangles(case):
    xy, tri = _square_mesh()
    kw = {}
    if case == "clockwise":
        tri = tri[:, ::-1].copy()
    elif case == "node-range":
        tri[1, 2] = 7
    elif case == "triple-edge":
        xy = np.vstack([xy, [[2.0, 0.5]], [[0.5, -1.0]]])
        tri = np.array([[0, 1, 2], [0, 2, 3], [1, 4, 2], [0, 5, 1], [1, 5, 4]], dtype=np.int32)
        # edge (1, 2) is used by three triangles once a duplicate is added
        tri = np.vstack([tri, [[2, 1, 4]]]).astype(np.int32)
    elif case == "two-layer-tracer":
        kw = dict(nlayers=2, ntracers=1, r=0.9)
    elif case == "bad-r":
        kw = dict(nlayers=2, r=1.0)
    d, keep = swe.mesh_desc(kind="tri", node_xy=xy, tri=tri, **kw)
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL


def test_null_handles_are_safe():
    assert swe.swe_nvars(None) == -1
    assert swe.swe_ncells(None) == -1
    assert swe.swe_path(None) == -1
    assert swe.swe_describe(None) == ""
    swe.swe_destroy(None)
    assert swe._lib.swe_step(None, 1, 0.5, None, None) == swe.SWE_E_INVAL
    assert swe._lib.swe_create_mesh(None, None) == swe.SWE_E_INVAL


def test_product_path_has_no_oracle_or_cpu_fallback():
    # the package never imports the oracle and never carries a CPU stepper
    pkg = os.path.join(ROOT, "finite_volume_shallow_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "swe_oracle" not in text, f


def test_bench_names_every_workload_with_its_precision():
    import inputs
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))
    import bench
    assert list(bench.WORKLOADS) == list(inputs.WORKLOADS) == list(bench.PRECISION)
    small = {"dam-break-64": dict(nx=8, ny=8), "hump-1024": dict(n=16), "flow-4096": dict(nx=16, ny=16),
             "tri-2M": dict(nq=4), "two-layer-1M": dict(nq=4)}
    for name, kw in small.items():
        assert inputs.make_workload(name, **kw).precision == bench.PRECISION[name], name


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    root = os.path.join(os.path.dirname(__file__), "..")
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


@pytest.mark.parametrize("kw, msg", [
    (dict(kind="tri", node_xy=np.zeros((3, 2)), tri=np.zeros((0, 3), dtype=np.int32)), "empty"),
    # the fused grid kernel addresses a field with 32-bit byte offsets
    (dict(kind="cart", nx=70000, ny=70000, dx=1.0, dy=1.0, precision="f32"), "too large"),
    (dict(kind="cart", nx=40000, ny=40000, dx=1.0, dy=1.0, precision="f64"), "too large"),
])
def test_create_rejects_empty_and_oversized_meshes(kw, msg):
    d, keep = swe.mesh_desc(**kw)
    with pytest.raises(swe.SweError) as e:
        swe.swe_create_mesh(d)
    assert e.value.status == swe.SWE_E_INVAL and msg in str(e.value)
