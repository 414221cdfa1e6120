"""Thin Python binding of libswe.so, the MI355X shallow-water step library.

Argument marshalling only: every step of the method runs in the HIP kernels
behind the C ABI declared in ``include/swe.h``.  The functions keep the C
names.  Host arrays are numpy float64; the ``*_device`` variants take torch
tensors (or raw device pointers) of the context's precision.

There is no fallback: if the compiled library is missing, importing this
module raises ``ImportError`` (run ``finite_volume_shallow_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswe.so")

SWE_ABI_VERSION = 2
SWE_OK, SWE_E_INVAL, SWE_E_NOMEM, SWE_E_HIP, SWE_E_NOSTATE = 0, -1, -2, -3, -4
SWE_E_DEPTH, SWE_E_NONFINITE, SWE_E_NONHYPERBOLIC = -5, -6, -7
SWE_MESH_CART, SWE_MESH_TRI = 0, 1
SWE_F64, SWE_F32 = 0, 1
SWE_BC_WALL, SWE_BC_PERIODIC = 0, 1
SWE_PATH_AUTO, SWE_PATH_EDGE, SWE_PATH_FUSED, SWE_PATH_RECOMPUTE = 0, 1, 2, 3
SWE_SCHEME_IR_ROE, SWE_SCHEME_ROE = 0, 1
SWE_ENTROPY_FIX_NONE, SWE_ENTROPY_FIX_HH = 0, 1

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)


class swe_mesh_desc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("mesh_kind", ctypes.c_int32),
        ("nlayers", ctypes.c_int32), ("ntracers", ctypes.c_int32),
        ("precision", ctypes.c_int32), ("path", ctypes.c_int32),
        ("scheme", ctypes.c_int32), ("entropy_fix", ctypes.c_int32),
        ("g", ctypes.c_double), ("r", ctypes.c_double),
        ("nx", ctypes.c_int64), ("ny", ctypes.c_int64),
        ("dx", ctypes.c_double), ("dy", ctypes.c_double),
        ("bc_x", ctypes.c_int32), ("bc_y", ctypes.c_int32),
        ("nnodes", ctypes.c_int64), ("ncells", ctypes.c_int64),
        ("node_xy", _D), ("tri", _I32), ("hip_stream", ctypes.c_void_p),
    ]


SWE_NOALLOC_MAX_STEPS = 1024

EXPORTS = ["swe_create_mesh", "swe_set_state", "swe_set_state_device", "swe_step", "swe_step_noalloc",
           "swe_get_state", "swe_get_state_device", "swe_get_dt_history", "swe_destroy",
           "swe_strerror", "swe_last_error", "swe_nvars", "swe_ncells", "swe_path",
           "swe_describe"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run finite_volume_shallow_amd/build.py")
    # torch carries its own HIP runtime (same soname); loading it first makes
    # libswe.so bind to that one runtime, so streams and device pointers
    # created through torch are valid in the library and vice versa.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    L.swe_create_mesh.argtypes = [ctypes.POINTER(swe_mesh_desc), ctypes.POINTER(P)]
    L.swe_create_mesh.restype = ctypes.c_int
    L.swe_set_state.argtypes = [P, _D, ctypes.POINTER(_D)]
    L.swe_set_state_device.argtypes = [P, P, ctypes.POINTER(P)]
    L.swe_step.argtypes = [P, ctypes.c_int32, ctypes.c_double, _D, _D]
    L.swe_step_noalloc.argtypes = [P, ctypes.c_int32, ctypes.c_double, _D, _D]
    L.swe_get_state.argtypes = [P, ctypes.POINTER(_D)]
    L.swe_get_state_device.argtypes = [P, ctypes.POINTER(P)]
    L.swe_get_dt_history.argtypes = [P, _D, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    L.swe_destroy.argtypes = [P]
    L.swe_destroy.restype = None
    L.swe_strerror.argtypes = [ctypes.c_int]
    L.swe_strerror.restype = ctypes.c_char_p
    L.swe_last_error.argtypes = [P]
    L.swe_last_error.restype = ctypes.c_char_p
    L.swe_nvars.argtypes = [P]
    L.swe_ncells.argtypes = [P]
    L.swe_ncells.restype = ctypes.c_int64
    L.swe_path.argtypes = [P]
    L.swe_describe.argtypes = [P]
    L.swe_describe.restype = ctypes.c_char_p
    return L


_lib = _load()


class SweError(RuntimeError):
    def __init__(self, status, detail=""):
        msg = _lib.swe_strerror(status).decode()
        super().__init__(f"swe status {status}: {msg}" + (f" ({detail})" if detail else ""))
        self.status = status


def _check(status, ctx=None):
    if status != SWE_OK:
        raise SweError(status, _lib.swe_last_error(ctx).decode())


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _expect_fields(ctx, arrays, what):
    """The library reads or writes ncells values per array and one array
    per conserved variable: check the caller's arrays before handing them
    over (raw device pointers cannot be checked and are passed as given)."""
    n, nv = _lib.swe_ncells(ctx), _lib.swe_nvars(ctx)
    if n < 0 or nv <= 0:
        raise ValueError(f"{what}: not a valid context")
    if len(arrays) != nv:
        raise ValueError(f"{what}: {nv} arrays expected, got {len(arrays)}")
    for a in arrays:
        size = a.numel() if hasattr(a, "numel") else (np.size(a) if isinstance(a, np.ndarray) else None)
        if size is not None and size != n:
            raise ValueError(f"{what}: arrays of {n} cells expected, got {size}")
        if hasattr(a, "is_contiguous") and not a.is_contiguous():
            raise ValueError(f"{what}: device tensors must be contiguous")


# ------------------------------------------------------------------ C names

def swe_create_mesh(desc: swe_mesh_desc):
    """Returns an opaque context handle (ctypes.c_void_p); keep ``desc``'s
    arrays alive only for the duration of this call."""
    ctx = ctypes.c_void_p()
    _check(_lib.swe_create_mesh(ctypes.byref(desc), ctypes.byref(ctx)))
    return ctx


def swe_set_state(ctx, z_bed, cons):
    z = _f64(z_bed)
    arrs = [_f64(a) for a in cons]
    _expect_fields(ctx, arrs, "swe_set_state")
    if z.size != _lib.swe_ncells(ctx):
        raise ValueError(f"swe_set_state: z_bed of {_lib.swe_ncells(ctx)} cells expected, got {z.size}")
    ptrs = (_D * len(arrs))(*[a.ctypes.data_as(_D) for a in arrs])
    _check(_lib.swe_set_state(ctx, z.ctypes.data_as(_D), ptrs), ctx)


def _devptr(x):
    return ctypes.c_void_p(x.data_ptr() if hasattr(x, "data_ptr") else int(x))


def swe_set_state_device(ctx, z_bed, cons):
    _expect_fields(ctx, list(cons), "swe_set_state_device")
    if hasattr(z_bed, "numel") and z_bed.numel() != _lib.swe_ncells(ctx):
        raise ValueError(f"swe_set_state_device: z_bed of {_lib.swe_ncells(ctx)} cells expected")
    ptrs = (ctypes.c_void_p * len(cons))(*[_devptr(a) for a in cons])
    _check(_lib.swe_set_state_device(ctx, _devptr(z_bed), ptrs), ctx)


def swe_step(ctx, nsteps, cfl):
    """Returns (t_advanced, last_dt); raises SweError on a failed batch."""
    t = ctypes.c_double()
    d = ctypes.c_double()
    _check(_lib.swe_step(ctx, int(nsteps), float(cfl), ctypes.byref(t), ctypes.byref(d)), ctx)
    return t.value, d.value


def swe_step_noalloc(ctx, nsteps, cfl):
    """swe_step without any allocation (at most SWE_NOALLOC_MAX_STEPS steps);
    returns (t_advanced, last_dt)."""
    t = ctypes.c_double()
    d = ctypes.c_double()
    _check(_lib.swe_step_noalloc(ctx, int(nsteps), float(cfl), ctypes.byref(t), ctypes.byref(d)), ctx)
    return t.value, d.value


def swe_get_state(ctx):
    n = _lib.swe_ncells(ctx)
    nv = _lib.swe_nvars(ctx)
    outs = [np.empty(n, dtype=np.float64) for _ in range(nv)]
    ptrs = (_D * nv)(*[a.ctypes.data_as(_D) for a in outs])
    _check(_lib.swe_get_state(ctx, ptrs), ctx)
    return outs


def swe_get_state_device(ctx, outs):
    _expect_fields(ctx, list(outs), "swe_get_state_device")
    ptrs = (ctypes.c_void_p * len(outs))(*[_devptr(a) for a in outs])
    _check(_lib.swe_get_state_device(ctx, ptrs), ctx)


def swe_get_dt_history(ctx):
    cnt = ctypes.c_int64()
    _check(_lib.swe_get_dt_history(ctx, None, 0, ctypes.byref(cnt)), ctx)
    out = np.empty(max(cnt.value, 1), dtype=np.float64)
    _check(_lib.swe_get_dt_history(ctx, out.ctypes.data_as(_D), cnt.value, ctypes.byref(cnt)), ctx)
    return out[:cnt.value]


def swe_destroy(ctx):
    _lib.swe_destroy(ctx)


def swe_strerror(status):
    return _lib.swe_strerror(status).decode()


def swe_last_error(ctx):
    return _lib.swe_last_error(ctx).decode()


def swe_nvars(ctx):
    return _lib.swe_nvars(ctx)


def swe_ncells(ctx):
    return _lib.swe_ncells(ctx)


def swe_path(ctx):
    return _lib.swe_path(ctx)


def swe_describe(ctx):
    return _lib.swe_describe(ctx).decode()


# ------------------------------------------------------------------ helpers

def mesh_desc(*, kind, nlayers=1, ntracers=0, precision="f64", path=SWE_PATH_AUTO,
              scheme="ir", entropy_fix=0, g=9.81, r=0.0, nx=0, ny=0, dx=0.0, dy=0.0, bc_x="wall", bc_y="wall",
              node_xy=None, tri=None, stream=None):
    """Fill a swe_mesh_desc.  Returns (desc, keepalive) - keep the second
    value referenced until swe_create_mesh returned."""
    for name, val, allowed in (("kind", kind, ("cart", "tri")), ("precision", precision, ("f32", "f64")),
                               ("bc_x", bc_x, ("wall", "periodic")), ("bc_y", bc_y, ("wall", "periodic"))):
        if val not in allowed:
            raise ValueError(f"{name} must be one of {allowed}, got {val!r}")
    d = swe_mesh_desc()
    d.abi_version = SWE_ABI_VERSION
    d.mesh_kind = SWE_MESH_CART if kind == "cart" else SWE_MESH_TRI
    d.nlayers = nlayers
    d.ntracers = ntracers
    d.precision = SWE_F32 if precision == "f32" else SWE_F64
    d.path = path
    if scheme not in ("ir", "classical"):
        raise ValueError(f"unknown scheme {scheme!r}")
    d.scheme = SWE_SCHEME_ROE if scheme == "classical" else SWE_SCHEME_IR_ROE
    d.entropy_fix = int(entropy_fix)
    d.g = g
    d.r = r
    keep = []
    if kind == "cart":
        d.nx, d.ny, d.dx, d.dy = nx, ny, dx, dy
        d.bc_x = SWE_BC_PERIODIC if bc_x == "periodic" else SWE_BC_WALL
        d.bc_y = SWE_BC_PERIODIC if bc_y == "periodic" else SWE_BC_WALL
    else:
        xy = _f64(node_xy).reshape(-1)
        t = np.ascontiguousarray(tri, dtype=np.int32).reshape(-1)
        keep += [xy, t]
        d.nnodes = xy.size // 2
        d.ncells = t.size // 3
        d.node_xy = xy.ctypes.data_as(_D)
        d.tri = t.ctypes.data_as(_I32)
    if stream is not None:
        d.hip_stream = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return d, keep


def desc_from_workload(w, path=SWE_PATH_AUTO, stream=None, precision=None):
    """Mesh description of an object with the fields of a workload record
    (kind, nlayers, ntracers, precision, g, r, nx, ny, dx, dy, bc_x, bc_y,
    node_xy, tri, and optionally scheme and entropy_fix)."""
    return mesh_desc(kind=w.kind, nlayers=w.nlayers, ntracers=w.ntracers,
                     precision=precision or w.precision, path=path,
                     scheme=getattr(w, "scheme", "ir"), entropy_fix=getattr(w, "entropy_fix", 0),
                     g=w.g, r=w.r,
                     nx=w.nx, ny=w.ny, dx=w.dx, dy=w.dy, bc_x=w.bc_x, bc_y=w.bc_y,
                     node_xy=w.node_xy, tri=w.tri, stream=stream)


class Context:
    """Owning wrapper of a context handle (destroyed on close / GC)."""

    def __init__(self, desc):
        self.ctx = swe_create_mesh(desc)

    def close(self):
        if self.ctx is not None and self.ctx.value:
            swe_destroy(self.ctx)
        self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()
