"""Python face of the plain fp64 CPU oracle (``swe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it to judge the GPU library.  The library itself never
imports, links or calls anything here.

Every entry point takes a :class:`inputs.Workload` (or raw edge states) and
works on float64 copies; nothing is shared with the GPU path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

OR_CODES = {0: "ok", 1: "bad mesh", 2: "depth <= 0", 3: "non-finite state",
            4: "non-hyperbolic Roe matrix", 5: "out of memory",
            6: "eigenvalue iteration did not converge"}

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle: {OR_CODES.get(code, code)}")
        self.code = code


def lib():
    """The compiled oracle.  SWE_ORACLE_LIB names another build of it (the
    planted-mistake check of the tests loads deliberately broken copies)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SWE_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.or_roe1_edge.argtypes = [_D, _D, ctypes.c_double, _D, _D]
        L.or_roe1c_edge.argtypes = [_D, _D, ctypes.c_double, _D, _D]
        L.or_roe1_edge_fix.argtypes = [_D, _D, ctypes.c_double, ctypes.c_int, _D, _D]
        L.or_roe1c_edge_fix.argtypes = [_D, _D, ctypes.c_double, ctypes.c_int, _D, _D]
        L.or_roe1_wall.argtypes = [_D, ctypes.c_double, _D, _D]
        L.or_roe2_edge.argtypes = [_D, _D, ctypes.c_double, ctypes.c_double, _D, _D, _D]
        L.or_roe2_wall.argtypes = [_D, ctypes.c_double, ctypes.c_double, _D, _D]
        L.or_roe2c_edge.argtypes = [_D, _D, ctypes.c_double, ctypes.c_double, _D, _D, _D]
        L.or_run_cart.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                  _D, _D, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.or_run_tri.argtypes = [ctypes.c_int64, _D, ctypes.c_int64, _I32,
                                 ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                 _D, _D, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.or_run_tri2.argtypes = [ctypes.c_int64, _D, ctypes.c_int64, _I32,
                                  ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_int, _D, _D, _D, _D, _D, _D, _D, _D,
                                  ctypes.c_int, ctypes.c_int]
        L.or_tri_geometry.argtypes = [ctypes.c_int64, _D, ctypes.c_int64, _I32,
                                      _I64, _D, _D, _D, _D]
        _lib = L
    return _lib


def _dp(a):
    return a.ctypes.data_as(_D) if a is not None else None


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64).copy()


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- edge level

def roe1_edge(L, R, g=9.81):
    """Flux leaving L for one-layer edge states (h, qn, qt, hc, H)."""
    L = _f64(L); R = _f64(R)
    phi = np.zeros(4); sp = ctypes.c_double()
    st = lib().or_roe1_edge(_dp(L), _dp(R), g, _dp(phi), ctypes.byref(sp))
    if st:
        raise OracleError(st)
    return phi, sp.value


def roe1_edge_fix(L, R, g=9.81, fix=1):
    """As roe1_edge, with the Harten-Hyman entropy fix (fix=1)."""
    L = _f64(L); R = _f64(R)
    phi = np.zeros(4); sp = ctypes.c_double()
    st = lib().or_roe1_edge_fix(_dp(L), _dp(R), g, int(fix), _dp(phi), ctypes.byref(sp))
    if st:
        raise OracleError(st)
    return phi, sp.value


def roe1c_edge_fix(L, R, g=9.81, fix=1):
    """As roe1c_edge, with the Harten-Hyman entropy fix (fix=1)."""
    L = _f64(L); R = _f64(R)
    phi = np.zeros(4); sp = ctypes.c_double()
    st = lib().or_roe1c_edge_fix(_dp(L), _dp(R), g, int(fix), _dp(phi), ctypes.byref(sp))
    if st:
        raise OracleError(st)
    return phi, sp.value


def roe1c_edge(L, R, g=9.81):
    """Classical Roe flux (four waves, contact waves for the transverse
    momentum and the pollutant) leaving L for one-layer edge states."""
    L = _f64(L); R = _f64(R)
    phi = np.zeros(4); sp = ctypes.c_double()
    st = lib().or_roe1c_edge(_dp(L), _dp(R), g, _dp(phi), ctypes.byref(sp))
    if st:
        raise OracleError(st)
    return phi, sp.value


def roe1_wall(L, g=9.81):
    L = _f64(L)
    phi = np.zeros(4); sp = ctypes.c_double()
    st = lib().or_roe1_wall(_dp(L), g, _dp(phi), ctypes.byref(sp))
    if st:
        raise OracleError(st)
    return phi, sp.value


def roe2_edge(L, R, g=9.81, r=0.98):
    """Two-layer edge flux for states (h1, q1n, q1t, h2, q2n, q2t, H).

    Returns (phi[6], speed, eigenvalues ascending[4])."""
    L = _f64(L); R = _f64(R)
    phi = np.zeros(6); lam = np.zeros(4); sp = ctypes.c_double()
    st = lib().or_roe2_edge(_dp(L), _dp(R), g, r, _dp(phi), ctypes.byref(sp), _dp(lam))
    if st:
        raise OracleError(st)
    return phi, sp.value, lam


def roe2c_edge(L, R, g=9.81, r=0.98):
    """Classical Roe flux of two layers (full 6x6 Roe matrix), states and
    results as roe2_edge."""
    L = _f64(L); R = _f64(R)
    phi = np.zeros(6); lam = np.zeros(4); sp = ctypes.c_double()
    st = lib().or_roe2c_edge(_dp(L), _dp(R), g, r, _dp(phi), ctypes.byref(sp), _dp(lam))
    if st:
        raise OracleError(st)
    return phi, sp.value, lam


def roe2_wall(L, g=9.81, r=0.98):
    L = _f64(L)
    phi = np.zeros(6); sp = ctypes.c_double()
    st = lib().or_roe2_wall(_dp(L), g, r, _dp(phi), ctypes.byref(sp))
    if st:
        raise OracleError(st)
    return phi, sp.value


def tri_geometry(node_xy, tri):
    xy = _f64(node_xy).ravel()
    t = np.ascontiguousarray(tri, dtype=np.int32).ravel()
    n = t.size // 3
    nb = np.zeros(3 * n, dtype=np.int64)
    ex = np.zeros(3 * n); ey = np.zeros(3 * n); ln = np.zeros(3 * n); ar = np.zeros(n)
    st = lib().or_tri_geometry(xy.size // 2, _dp(xy), n, t.ctypes.data_as(_I32),
                               nb.ctypes.data_as(_I64), _dp(ex), _dp(ey), _dp(ln), _dp(ar))
    if st:
        raise OracleError(st)
    return (nb.reshape(n, 3), ex.reshape(n, 3), ey.reshape(n, 3),
            ln.reshape(n, 3), ar)


# ---------------------------------------------------------------- time loop

def run(w, nsteps=None, nthreads=None, check=True):
    """Advance a Workload by nsteps steps (default w.nsteps).

    Returns (state list, dts array, status).  Raises OracleError when
    ``check`` and the run failed."""
    nsteps = w.nsteps if nsteps is None else nsteps
    nthreads = default_threads() if nthreads is None else nthreads
    st_arrays = [_f64(a) for a in w.state]
    z = _f64(w.z)
    dts = np.zeros(max(nsteps, 1))
    L = lib()
    classical = int(getattr(w, "scheme", "ir") == "classical")
    fix = int(getattr(w, "entropy_fix", 0))
    if fix and w.nlayers != 1:
        raise ValueError("the entropy fix is implemented for one layer")
    if classical and w.kind == "cart" and w.nlayers != 1:
        raise ValueError("two layers run on triangle meshes only")
    if w.kind == "cart":
        hc = st_arrays[3] if w.ntracers else None
        status = L.or_run_cart(w.nx, w.ny, w.dx, w.dy, int(w.bc_x == "periodic"),
                               int(w.bc_y == "periodic"), w.g, w.cfl, nsteps,
                               _dp(z), _dp(st_arrays[0]), _dp(st_arrays[1]),
                               _dp(st_arrays[2]), _dp(hc), _dp(dts), nthreads, classical, fix)
    elif w.nlayers == 1:
        xy = _f64(w.node_xy).ravel()
        t = np.ascontiguousarray(w.tri, dtype=np.int32).ravel()
        hc = st_arrays[3] if w.ntracers else None
        status = L.or_run_tri(xy.size // 2, _dp(xy), t.size // 3, t.ctypes.data_as(_I32),
                              w.g, w.cfl, nsteps, _dp(z), _dp(st_arrays[0]),
                              _dp(st_arrays[1]), _dp(st_arrays[2]), _dp(hc), _dp(dts),
                              nthreads, classical, fix)
    else:
        xy = _f64(w.node_xy).ravel()
        t = np.ascontiguousarray(w.tri, dtype=np.int32).ravel()
        status = L.or_run_tri2(xy.size // 2, _dp(xy), t.size // 3, t.ctypes.data_as(_I32),
                               w.g, w.r, w.cfl, nsteps, _dp(z),
                               *[_dp(a) for a in st_arrays], _dp(dts), nthreads, classical)
    if check and status:
        raise OracleError(status)
    return st_arrays, dts[:nsteps], status
