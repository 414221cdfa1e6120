"""Seeded generators for the five shallow-water workloads.

Each generator returns a :class:`Workload`: the mesh (a Cartesian grid or a
triangle list), the bed elevation ``z`` per cell and the initial conserved
state per cell.  Sizes default to the full workloads; smaller sizes keep the
same recipe on the same physical domain with coarser cells, so a test case
at 128x128 is a low-resolution copy of the 1024x1024 case.

Conventions (shared by every consumer, stated once here):

* Cartesian cell ``k = j * nx + i``; cell centre ``((i + 0.5) dx, (j + 0.5) dy)``.
* Triangles are listed counter-clockwise as three node ids.
* A one-layer state is ``[h, qx, qy]`` plus ``[hc]`` when a pollutant is
  carried (``hc`` = depth times concentration).  A two-layer state is
  ``[h1, q1x, q1y, h2, q2x, q2y]`` with layer 1 on top.
* ``z`` is the bed elevation; the depth function of the two-layer model
  is ``H = -z`` (only differences of ``H`` enter the scheme).
* Random draws come from ``numpy.random.default_rng(seed)`` with a fixed
  seed per workload (1001 ... 1005, the default of each generator's ``seed``)
  in the fixed order written in each generator.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

G = 9.81


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                      # "cart" or "tri"
    nlayers: int
    ntracers: int
    precision: str                 # "f64" or "f32"
    g: float
    r: float
    cfl: float
    nsteps: int
    z: np.ndarray
    state: list
    # Cartesian grids
    nx: int = 0
    ny: int = 0
    dx: float = 0.0
    dy: float = 0.0
    bc_x: str = "wall"
    bc_y: str = "wall"
    # triangle meshes
    node_xy: np.ndarray | None = None
    tri: np.ndarray | None = None
    # "ir" (the IR-Roe scheme) or "classical" (full Roe matrix)
    scheme: str = "ir"
    # 1: Harten-Hyman entropy fix (one layer)
    entropy_fix: int = 0

    @property
    def ncells(self) -> int:
        return int(self.z.shape[0])

    @property
    def nvars(self) -> int:
        return 6 if self.nlayers == 2 else 3 + self.ntracers

    def copy(self, **changes) -> "Workload":
        w = dataclasses.replace(self, **changes)
        w.z = np.array(w.z, copy=True)
        w.state = [np.array(a, copy=True) for a in w.state]
        return w


def round_to_f32(w: Workload) -> Workload:
    """The same workload with bed and state rounded through float32.

    A float32 run starts from these values, so a float64 reference that is
    compared with it must start from them too.
    """
    r = w.copy(precision="f32")
    r.z = r.z.astype(np.float32).astype(np.float64)
    r.state = [a.astype(np.float32).astype(np.float64) for a in r.state]
    return r


# ----------------------------------------------------------------------------
# shared pieces of the recipes (pure input construction)
# ----------------------------------------------------------------------------

def _gauss_sum_grid(xc, yc, amps, sigmas, cx, cy, x_period=None):
    """Sum of isotropic Gaussians a*exp(-|x-x0|^2/(2 s^2)) on a tensor grid.

    Each Gaussian separates into a y factor times an x factor, so the sum is
    the product of a (ny, k) and a (k, nx) matrix."""
    shifts = [0.0] if x_period is None else [-x_period, 0.0, x_period]
    amps = np.asarray(amps)[:, None]
    sig = np.asarray(sigmas)[:, None]
    gy = np.exp(-((yc[None, :] - np.asarray(cy)[:, None]) ** 2) / (2.0 * sig * sig))
    gx = np.zeros((len(amps), xc.size))
    for sh in shifts:
        gx += np.exp(-((xc[None, :] - np.asarray(cx)[:, None] - sh) ** 2) / (2.0 * sig * sig))
    return (gy * amps).T @ gx


def _gauss_sum_points(px, py, amps, sigmas, cx, cy):
    out = np.zeros_like(px)
    for a, s, x0, y0 in zip(amps, sigmas, cx, cy):
        out += a * np.exp(-((px - x0) ** 2 + (py - y0) ** 2) / (2.0 * s * s))
    return out


def _part1by1(v):
    v = v.astype(np.uint64) & np.uint64(0xFFFF)
    v = (v | (v << np.uint64(8))) & np.uint64(0x00FF00FF)
    v = (v | (v << np.uint64(4))) & np.uint64(0x0F0F0F0F)
    v = (v | (v << np.uint64(2))) & np.uint64(0x33333333)
    v = (v | (v << np.uint64(1))) & np.uint64(0x55555555)
    return v


def morton_order(px, py):
    """Stable order of points by the 2x16-bit Morton code of their position."""
    x0, x1 = px.min(), px.max()
    y0, y1 = py.min(), py.max()
    qx = np.floor((px - x0) / max(x1 - x0, 1e-300) * 65535.0).astype(np.int64)
    qy = np.floor((py - y0) / max(y1 - y0, 1e-300) * 65535.0).astype(np.int64)
    code = _part1by1(qx) | (_part1by1(qy) << np.uint64(1))
    return np.argsort(code, kind="stable")


def lattice_triangles(nq, rng, spacing=1.0, jitter=0.2, morton=True):
    """Jittered quad lattice split into counter-clockwise triangles.

    Nodes sit on an (nq+1)^2 lattice of the given spacing; interior nodes
    move by independent uniform draws in [-jitter, jitter] * spacing (x draws
    for every node first, then y draws), boundary nodes stay put.  Each quad
    (i, j) is split along its (i, j)-(i+1, j+1) diagonal.  With ``morton`` the
    triangles are sorted by the Morton code of their centroids.
    Returns node_xy (nnodes, 2) float64 and tri (ncells, 3) int32.
    """
    n1 = nq + 1
    ii, jj = np.meshgrid(np.arange(n1), np.arange(n1))
    ii = ii.ravel()
    jj = jj.ravel()
    x = ii * spacing
    y = jj * spacing
    jx = rng.uniform(-jitter, jitter, n1 * n1) * spacing
    jy = rng.uniform(-jitter, jitter, n1 * n1) * spacing
    interior = (ii > 0) & (ii < nq) & (jj > 0) & (jj < nq)
    x = x + np.where(interior, jx, 0.0)
    y = y + np.where(interior, jy, 0.0)
    node_xy = np.stack([x, y], axis=1)

    qi, qj = np.meshgrid(np.arange(nq), np.arange(nq))
    qi = qi.ravel()
    qj = qj.ravel()
    n00 = qj * n1 + qi
    n10 = n00 + 1
    n01 = n00 + n1
    n11 = n01 + 1
    t1 = np.stack([n00, n10, n11], axis=1)
    t2 = np.stack([n00, n11, n01], axis=1)
    tri = np.empty((2 * nq * nq, 3), dtype=np.int64)
    tri[0::2] = t1
    tri[1::2] = t2
    if morton:
        cx, cy = triangle_centroids(node_xy, tri)
        tri = tri[morton_order(cx, cy)]
    return node_xy, tri.astype(np.int32)


def triangle_centroids(node_xy, tri):
    p = node_xy[tri]
    return p[:, :, 0].mean(axis=1), p[:, :, 1].mean(axis=1)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

def dam_break(nx=64, ny=64, nsteps=100):
    """Dam break with pollutant on a flat bed, 1 m square cells, walls.

    Depth 2 and concentration 1 for cell centres x < nx/2, else depth 1 and
    concentration 0; at rest.
    """
    i = np.arange(nx)
    left = (i + 0.5) < nx / 2.0
    h_row = np.where(left, 2.0, 1.0)
    c_row = np.where(left, 1.0, 0.0)
    h = np.tile(h_row, ny)
    hc = np.tile(h_row * c_row, ny)
    z = np.zeros(nx * ny)
    zero = np.zeros(nx * ny)
    return Workload(
        name=f"dam-break {nx}x{ny} + pollutant", kind="cart", nlayers=1,
        ntracers=1, precision="f64", g=G, r=0.0, cfl=0.9, nsteps=nsteps,
        z=z, state=[h, zero.copy(), zero.copy(), hc], nx=nx, ny=ny,
        dx=1.0, dy=1.0, bc_x="wall", bc_y="wall")


def gaussian_hump(n=1024, nsteps=1000, precision="f64", seed=1002, hump=True,
            blob=True):
    """Gaussian hump over a 16-Gaussian bed (lake at rest at 5 m).

    The domain is 1024 m square; n cells per side (1 m cells at n = 1024).
    Draw order: 16 amplitudes U[0.1, 0.8] m, 16 sigmas U[20, 120] m,
    16 centre x, 16 centre y (uniform over the domain), then the hump centre
    (uniform in the central half).  Depth h = 5 - z + 0.5 exp(-r^2/(2*30^2));
    pollutant concentration 1 within 50 m of the hump centre.
    """
    L = 1024.0
    dx = L / n
    rng = np.random.default_rng(seed)
    amps = rng.uniform(0.1, 0.8, 16)
    sig = rng.uniform(20.0, 120.0, 16)
    cx = rng.uniform(0.0, L, 16)
    cy = rng.uniform(0.0, L, 16)
    hx, hy = rng.uniform(256.0, 768.0, 2)
    xc = (np.arange(n) + 0.5) * dx
    yc = (np.arange(n) + 0.5) * dx
    z = _gauss_sum_grid(xc, yc, amps, sig, cx, cy)
    r2 = (xc[None, :] - hx) ** 2 + (yc[:, None] - hy) ** 2
    h = 5.0 - z
    if hump:
        h = h + 0.5 * np.exp(-r2 / (2.0 * 30.0 ** 2))
    c = (r2 <= 50.0 ** 2).astype(np.float64) if blob else np.zeros_like(h)
    zero = np.zeros(n * n)
    return Workload(
        name=f"gaussian-hump {n}x{n}", kind="cart", nlayers=1, ntracers=1,
        precision=precision, g=G, r=0.0, cfl=0.9, nsteps=nsteps,
        z=z.ravel(), state=[h.ravel(), zero.copy(), zero.copy(), (h * c).ravel()],
        nx=n, ny=n, dx=dx, dy=dx, bc_x="wall", bc_y="wall")


def _stream_modes(rng):
    a = rng.standard_normal((9, 8))
    m = np.arange(9)[:, None]
    nn = np.arange(1, 9)[None, :]
    a = a / (m * m + nn * nn)
    ph = rng.uniform(0.0, 2.0 * math.pi, (9, 8))
    return a, ph


def smooth_flow(nx=4096, ny=4096, nsteps=500, precision="f32", seed=1003,
            flat=False, still=False):
    """Smooth random flow over a 64-Gaussian bed on 20 m depth.

    Square cells of 40960/nx m (10 m at nx = 4096); the domain is nx by ny
    cells.  x periodic, walls in y.  Draw order: 64 amplitudes U[1, 5] m,
    64 sigmas U[300, 3000] m (30 to 300 cells of 10 m), 64 centre x, 64
    centre y; stream-function modes A_mn ~ N(0,1)/(m^2+n^2) (m = 0..8,
    n = 1..8) and phases U[0, 2pi); then the same for the concentration
    field.  psi = sum A sin(n pi y/Ly) cos(2 pi m x/Lx + phi); u = d psi/dy,
    v = -d psi/dx scaled to a maximum speed of 1 m/s.  Concentration =
    min-max scaled field of the same form.  Depth h = 20 - z.
    """
    dx = 40960.0 / nx
    Lx = nx * dx
    Ly = ny * dx
    rng = np.random.default_rng(seed)
    amps = rng.uniform(1.0, 5.0, 64)
    sig = rng.uniform(300.0, 3000.0, 64)
    cx = rng.uniform(0.0, Lx, 64)
    cy = rng.uniform(0.0, Ly, 64)
    a_u, ph_u = _stream_modes(rng)
    a_c, ph_c = _stream_modes(rng)
    X = (np.arange(nx) + 0.5) * dx
    Y = (np.arange(ny) + 0.5) * dx
    z = _gauss_sum_grid(X, Y, amps, sig, cx, cy, x_period=Lx)
    if flat:
        z = np.zeros_like(z)
    cos_y = np.empty((ny, 8))
    sin_y = np.empty((ny, 8))
    ux = np.zeros((8, nx))
    vx = np.zeros((8, nx))
    cxr = np.zeros((8, nx))
    for n in range(1, 9):
        ky = n * math.pi / Ly
        cos_y[:, n - 1] = np.cos(ky * Y)
        sin_y[:, n - 1] = np.sin(ky * Y)
        for m in range(9):
            kx = 2.0 * math.pi * m / Lx
            ux[n - 1] += a_u[m, n - 1] * ky * np.cos(kx * X + ph_u[m, n - 1])
            vx[n - 1] += a_u[m, n - 1] * kx * np.sin(kx * X + ph_u[m, n - 1])
            cxr[n - 1] += a_c[m, n - 1] * np.cos(kx * X + ph_c[m, n - 1])
    u = cos_y @ ux
    v = sin_y @ vx
    psi_c = sin_y @ cxr
    speed = np.sqrt(u * u + v * v).max()
    u /= speed
    v /= speed
    if still:
        u[:] = 0.0
        v[:] = 0.0
    c = (psi_c - psi_c.min()) / (psi_c.max() - psi_c.min())
    h = 20.0 - z
    return Workload(
        name=f"smooth-flow {nx}x{ny}", kind="cart", nlayers=1, ntracers=1,
        precision=precision, g=G, r=0.0, cfl=0.9, nsteps=nsteps,
        z=z.ravel(), state=[h.ravel(), (h * u).ravel(), (h * v).ravel(),
                            (h * c).ravel()],
        nx=nx, ny=ny, dx=dx, dy=dx, bc_x="periodic", bc_y="wall")


def circular_dam_break(nq=1000, nsteps=200, seed=1004, still=False):
    """Circular dam break on a jittered, Morton-ordered triangle mesh.

    The domain is 1000 m square, nq x nq quads (1 m at nq = 1000), each split
    into two triangles.  Draw order: node jitter (x then y), then the
    16-Gaussian bed of the 1024x1024 workload (amplitudes U[0.1, 0.8] m,
    sigmas U[20, 120] m, centres uniform), evaluated at the triangle
    centroids.  Depth 3 within 200 m of the domain centre, else 1; at rest;
    no pollutant.  ``still`` gives a lake at rest (h = 5 - z) instead.
    """
    L = 1000.0
    rng = np.random.default_rng(seed)
    node_xy, tri = lattice_triangles(nq, rng, spacing=L / nq)
    amps = rng.uniform(0.1, 0.8, 16)
    sig = rng.uniform(20.0, 120.0, 16)
    cx = rng.uniform(0.0, L, 16)
    cy = rng.uniform(0.0, L, 16)
    px, py = triangle_centroids(node_xy, tri)
    z = _gauss_sum_points(px, py, amps, sig, cx, cy)
    if still:
        h = 5.0 - z
    else:
        d = np.hypot(px - L / 2.0, py - L / 2.0)
        h = np.where(d < 200.0, 3.0, 1.0)
    zero = np.zeros_like(h)
    return Workload(
        name=f"circular-dam-break {tri.shape[0]} triangles", kind="tri",
        nlayers=1, ntracers=0, precision="f64", g=G, r=0.0, cfl=0.9,
        nsteps=nsteps, z=z, state=[h, zero.copy(), zero.copy()],
        node_xy=node_xy, tri=tri)


def two_layer_dam_break(nq=707, nsteps=200, seed=1005, step=True):
    """Two-layer internal dam break on a jittered triangle mesh.

    The domain is 707 m square, nq x nq quads (1 m at nq = 707).  Draw
    order: node jitter, the 16-Gaussian bed (as for the circular dam break), then the
    half-plane angle U[0, 2pi) and a point uniform in the central half of
    the domain.  At rest h1 = 2.5 and h2 = 2.5 - z; inside the half-plane
    the interface is raised by 0.5 m (h2 + 0.5, h1 - 0.5).  Density ratio
    0.98.
    """
    L = 707.0
    rng = np.random.default_rng(seed)
    node_xy, tri = lattice_triangles(nq, rng, spacing=L / nq)
    amps = rng.uniform(0.1, 0.8, 16)
    sig = rng.uniform(20.0, 120.0, 16)
    cx = rng.uniform(0.0, L, 16)
    cy = rng.uniform(0.0, L, 16)
    theta = rng.uniform(0.0, 2.0 * math.pi)
    p = rng.uniform(L / 4.0, 3.0 * L / 4.0, 2)
    px, py = triangle_centroids(node_xy, tri)
    z = _gauss_sum_points(px, py, amps, sig, cx, cy)
    h1 = np.full_like(z, 2.5)
    h2 = 2.5 - z
    if step:
        inside = (px - p[0]) * math.cos(theta) + (py - p[1]) * math.sin(theta) > 0
        h1 = np.where(inside, h1 - 0.5, h1)
        h2 = np.where(inside, h2 + 0.5, h2)
    zero = np.zeros_like(z)
    return Workload(
        name=f"two-layer internal dam break {tri.shape[0]} triangles",
        kind="tri", nlayers=2, ntracers=0, precision="f64", g=G, r=0.98,
        cfl=0.9, nsteps=nsteps, z=z,
        state=[h1, zero.copy(), zero.copy(), h2, zero.copy(), zero.copy()],
        node_xy=node_xy, tri=tri)


# the workloads by name (each at its full size by default)
WORKLOADS = {
    "dam-break-64": dam_break,
    "hump-1024": gaussian_hump,
    "flow-4096": smooth_flow,
    "tri-2M": circular_dam_break,
    "two-layer-1M": two_layer_dam_break,
}


def make_workload(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)
