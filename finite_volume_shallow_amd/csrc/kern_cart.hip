// Fused structured-grid path: one kernel launch per time step.
//
// [IR] Eq. (4) needs the global dt of the step before any cell can be
// updated, and dt comes from the wave speeds of the state at the start of
// the step (Eq. (5)).  Splitting the step at that dependency would cost a
// second pass over the state.  Instead the launch for step n
//   1. reads W^n on its tile plus a two-cell halo,
//   2. computes the Roe fluctuations of every edge it needs ([IR] Sec. 2.2,
//      one layer plus the upwinded pollutant of [MG]) and updates W^{n+1}
//      on the tile plus a one-cell ring, using dt^n reduced by the previous
//      launch,
//   3. forms the Eq. (5) wave speeds of W^{n+1} on the tile's edges and
//      folds the tile's minimum of 2 gamma |V| / sum |G| ||D|| into the
//      partial minima that the next launch reduces to dt^{n+1},
//   4. writes W^{n+1} of the tile (ping-pong buffers, no in-place hazard).
// The halo work (a one-cell ring of fluxes, a two-cell ring of loads) is
// the price of reading and writing the state exactly once per step.
//
// Work layout (CDNA 64-wide wavefronts): one wavefront per tile; a tile is
// 60 columns (lanes 2..61; lanes 0, 1, 62, 63 carry the halo columns) by
// TY rows.  The wavefront marches up its tile row by row: a row of every
// field is one coalesced load, the neighbour across an x-edge is the next
// lane (a DPP wave shift, no LDS), and the neighbour across a y-edge is the
// previous row, still in registers.  No LDS tile and no barrier are needed.
// Each edge is evaluated once per pass by the lane on its left (x) or by
// the row above it (y), and both cells take their part of it, as in the
// right/bottom-edge ownership of [MG]'s thread-block kernel.
//
// Per cell and row the lane prepares 1/h, sqrt(h) and the velocities once
// (one reciprocal square root), so an edge costs one reciprocal and one
// reciprocal square root on top of its arithmetic (fastmath.hpp: hardware
// approximations in float32, Newton-refined estimates in float64).
//
// dt: each wavefront min-reduces its candidates with shuffles and issues one
// atomic min (on the IEEE bits of a non-negative double) into one of 64
// partial slots; the next launch reads the 64 partials and reduces them in
// one wavefront.  Three slot banks rotate (read / written / cleared).
//
// Workgroup order is XCD-aware: workgroups are dealt round-robin to the
// eight XCDs, so tile t is mapped to a contiguous band of tiles per XCD and
// the wavefronts sharing halo rows and columns share one L2.
#include "dt_reduce.hpp"
#include "roe_device.hpp"
#include "swe_internal.hpp"

namespace swe {

constexpr int CART_LANES = 64;
constexpr int CART_COLS = 60; // useful columns per tile
constexpr int NUM_XCD = 8;
constexpr int NPART = 64;     // partial dt slots per bank

template <typename T, bool TR> struct CartArgs {
    const T *__restrict__ in0, *__restrict__ in1; // W^n: the record planes (cart_plane)
    const T *__restrict__ z;
    T *__restrict__ out0, *__restrict__ out1;     // W^{n+1}, planes as `in`
    int nx, ny, perx, pery;
    T dx, dy, g, cfl;
    int ty;        // rows per tile
    int alt;       // odd row blocks march downward
    int rev;       // tiles in reverse order (streaming mode, every other step)
    int nstrips;   // tiles across x
    int ntiles;    // tiles in total
    int per_xcd;   // tiles per XCD band
    double *part;  // [3][NPART] partial minima
    StepBook book;
    int64_t step;  // index of the step within the batch (dt history)
    int bank0;     // partial-minimum bank of the batch's first step
};

// ---------------------------------------------------------------- math

// ---------------------------------------------------------------- lane moves
// DPP wave shifts: wave_shl:1 gives lane i the value of lane i+1, wave_shr:1
// the value of lane i-1; the lane without a source (63, resp. 0) reads 0.
// Those two lanes are halo lanes whose own results are never used.
constexpr int DPP_WAVE_SHL1 = 0x130;
constexpr int DPP_WAVE_SHR1 = 0x138;

template <int CTRL> __device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ double dpp(double v)
{
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, true);
    return __hiloint2double(hi, lo);
}
template <typename T> __device__ __forceinline__ T nxt(T v) { return dpp<DPP_WAVE_SHL1>(v); }
template <typename T> __device__ __forceinline__ T prv(T v) { return dpp<DPP_WAVE_SHR1>(v); }

// ---------------------------------------------------------------- cells

// A cell of W^n with the per-cell quantities its edges share.
template <typename T> struct PC {
    T h, s, u, v, cc, qx, qy, c, z;
};

template <typename T> __device__ __forceinline__ PC<T> prep(T h, T qx, T qy, T c, T z)
{
    PC<T> p;
    p.h = h;
    p.qx = qx;
    p.qy = qy;
    p.c = c;
    p.z = z;
    const T r = FM<T>::rsq(h);
    p.s = h * r;
    const T ih = r * r;
    p.u = qx * ih;
    p.v = qy * ih;
    p.cc = c * ih;
    return p;
}

// One edge, in the edge frame.  Mass and normal momentum as fluctuations
// of its two cells (a: the cell on the normal's tail, b: its head), so that
// float32 keeps the differences exactly that the large hydrostatic terms
// would swamp; the transverse momentum and the pollutant as the flux through
// the edge (ft, fc), which both cells share (a cell's own-state terms cancel
// over its two edges of a direction, and these rows carry no hydrostatic
// term).
template <typename T> struct EF {
    T am, an, bm, bn, ft, fc;
};

// Interior edge, states given in the edge frame (qn, un normal; ut
// transverse).  [IR] Sec. 2.2 steps 1-3 with one layer: Roe averages,
// X = F(W_b) - F(W_a) - S dH, P^- X by the 2x2 eigen-decomposition,
// the transverse momentum and the pollutant upwinded by the mass flux.
// FX = FLUX_ROE: the classical Roe flux of the whole system instead, whose
// transverse momentum and pollutant rows are contact waves of speed ubar
// (Roe averages vbar, Cbar of the transverse velocity and the
// concentration, weighted by sqrt(h) like ubar).  FLUX_IR_HH / FLUX_ROE_HH:
// either with the Harten-Hyman entropy fix (hh_fix).
template <typename T, bool TR, int FX>
__device__ __forceinline__ EF<T> flux(T hL, T sL, T qL, T uL, T tL, T cL, T zL, T hR, T sR, T qR, T uR, T tR,
                                      T cR, T zR, T g)
{
    EF<T> o;
    const T isum = FM<T>::rcp(sL + sR);
    const T ubar = (sL * uL + sR * uR) * isum;
    const T c2 = g * T(0.5) * (hL + hR);
    const T irc = FM<T>::rsq(c2);
    const T c = c2 * irc;
    const T i2c = T(0.5) * irc;
    const T lam1 = ubar - c, lam2 = ubar + c;
    const T X0 = qR - qL;
    const T X1 = (qR * uR - qL * uL) + c2 * ((hR - hL) + (zR - zL));
    const T a1 = (lam2 * X0 - X1) * i2c;
    const T a2 = (X1 - lam1 * X0) * i2c;
    const T w1 = wminus(lam1), w2 = wminus(lam2);
    T pm0 = w1 * a1 + w2 * a2;
    T pm1 = w1 * a1 * lam1 + w2 * a2 * lam2;
    if (flux_hh(FX)) hh_fix(hL, qL, uL, hR, qR, uR, lam1, lam2, i2c, g, pm0, pm1);
    o.am = pm0;
    o.an = pm1;
    o.bm = X0 - pm0;
    o.bn = X1 - pm1;
    if (flux_classical(FX)) {
        // the contact waves: F_t(W_a) + (P^- X)_t
        const T wu = wminus(ubar);
        const T vbar = (sL * tL + sR * tR) * isum;
        const T Ft = qL * tL;
        o.ft = Ft + (vbar * pm0 + wu * ((qR * tR - Ft) - vbar * X0));
        if (TR) {
            const T cbar = (sL * cL + sR * cR) * isum;
            const T Fc = qL * cL;
            o.fc = Fc + (cbar * pm0 + wu * ((qR * cR - Fc) - cbar * X0));
        } else {
            o.fc = T(0);
        }
        return o;
    }
    // carried by the mass flux phi0, upwinded by its sign
    const T phi0 = qL + pm0;
    const bool up = phi0 > T(0);
    o.ft = phi0 * (up ? tL : tR);
    o.fc = TR ? phi0 * (up ? cL : cR) : T(0);
    return o;
}

// Reflective wall seen from the cell (edge frame, outward normal): the mass,
// transverse and pollutant fluxes are zero (the mass fluctuation is -qn and
// ft = fc = 0 at the wall), the normal momentum gets the mirror-problem term
// sqrt(g h) qn.
template <typename T> __device__ __forceinline__ void wall(T h, T qn, T g, T &m, T &n)
{
    m = -qn;
    n = FM<T>::sqrt(g * h) * qn;
}

// Eq. (5) speed |u_Roe| + c of an edge from per-cell s = sqrt(h) and
// a = qn / sqrt(h):  u_Roe = (a_L + a_R) / (s_L + s_R).
template <typename T> __device__ __forceinline__ T espeed(T hL, T sL, T aL, T hR, T sR, T aR, T g)
{
    return fabs((aL + aR) * FM<T>::rcp(sL + sR)) + FM<T>::sqrt(g * T(0.5) * (hL + hR));
}

// Element k of an array through a 32-bit byte offset (scalar base + vector
// offset addressing; grids on this path hold < 2^31 cells, < 2^32 bytes per
// float32 field, < 2^32 bytes per float64 field below 2^29 cells).
template <typename T> __device__ __forceinline__ const T &at(const T *base, uint32_t k)
{
    return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + (uint32_t)(k * (uint32_t)sizeof(T)));
}
template <typename T> __device__ __forceinline__ T &at(T *base, uint32_t k)
{
    return *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + (uint32_t)(k * (uint32_t)sizeof(T)));
}

// The state of a structured grid is stored interleaved, in planes of
// 16-byte records: float32 cells are one record (h, qx, qy, hc) (or
// (h, qx, qy), 12 bytes, without the pollutant); float64 cells are a record
// (h, qx) in plane 0 and (qy, hc) (or qy alone) in plane 1, which starts
// after the N records of plane 0.  A wavefront's row of a plane is one
// contiguous access (1 KB with 16-byte records) instead of a separate
// 256-byte (float32) or 512-byte (float64) piece per variable; the memory
// system serves the wide accesses markedly faster when thousands of
// wavefronts march different rows at once.  The bed z stays a plain array.
// cart_plane (host) lays out the same planes.
template <typename T, int W> struct CVec {
    typedef T V __attribute__((ext_vector_type(W)));
};

// Element k of plane `base` with W reals per record (W = 1, 2 or 4 load as
// one instruction; W = 3 as three adjacent reals), 32-bit byte offsets.
// NTL: a non-temporal load (compile-time, so that no optimisation can merge
// it with a plain load of the same address and drop the hint).
template <typename T, int W, bool NTL = false>
__device__ __forceinline__ void ld_w(const T *base, uint32_t k, T (&o)[W])
{
    const char *p = reinterpret_cast<const char *>(base) + (uint32_t)(k * (uint32_t)(W * sizeof(T)));
    if constexpr (W == 2 || W == 4) {
        typedef typename CVec<T, W>::V V;
        V v;
        if constexpr (NTL) v = __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
        else v = *reinterpret_cast<const V *>(p);
#pragma unroll
        for (int i = 0; i < W; ++i) o[i] = v[i];
    } else {
#pragma unroll
        for (int i = 0; i < W; ++i) {
            if constexpr (NTL) o[i] = __builtin_nontemporal_load(reinterpret_cast<const T *>(p) + i);
            else o[i] = reinterpret_cast<const T *>(p)[i];
        }
    }
}

// Streaming mode, for grids whose two state copies and bed exceed the
// last-level cache: W^n is loaded non-temporally (beyond the halo rows that
// a neighbouring tile reads at about the same time, the launch does not read
// it again), W^{n+1} is stored normally, and every other step runs its
// tiles in reverse order, so that a step starts with the state its
// predecessor wrote last, the part most likely still in the cache, and the
// bed stays there.  Non-temporal stores as well cost about 1 us more on the
// 4096^2 grid: the state they write is the next step's first read.  A grid
// that fits the cache keeps plain loads and the forward order, since it
// reads its state back from the cache in the next launch anyway.
template <typename T, int W> __device__ __forceinline__ void st_w(T *base, uint32_t k, const T (&x)[W])
{
    char *p = reinterpret_cast<char *>(base) + (uint32_t)(k * (uint32_t)(W * sizeof(T)));
    if constexpr (W == 2 || W == 4) {
        typedef typename CVec<T, W>::V V;
        V v;
#pragma unroll
        for (int i = 0; i < W; ++i) v[i] = x[i];
        *reinterpret_cast<V *>(p) = v;
    } else {
#pragma unroll
        for (int i = 0; i < W; ++i) reinterpret_cast<T *>(p)[i] = x[i];
    }
}

// Cell k of the state (NR = 3 or 4 variables) from / to its planes.
template <typename T, int NR, bool NTL = false>
__device__ __forceinline__ void ld_rec(const T *p0, const T *p1, uint32_t k, T &h, T &qx, T &qy, T &c)
{
    if constexpr (sizeof(T) == 4) {
        T a[NR];
        ld_w<T, NR, NTL>(p0, k, a);
        h = a[0];
        qx = a[1];
        qy = a[2];
        c = NR == 4 ? a[NR - 1] : T(0);
    } else {
        T a[2], b[NR - 2];
        ld_w<T, 2, NTL>(p0, k, a);
        ld_w<T, NR - 2, NTL>(p1, k, b);
        h = a[0];
        qx = a[1];
        qy = b[0];
        c = NR == 4 ? b[NR - 3] : T(0);
    }
}
template <typename T, int NR>
__device__ __forceinline__ void st_rec(T *p0, T *p1, uint32_t k, T h, T qx, T qy, T c)
{
    if constexpr (sizeof(T) == 4) {
        T a[NR];
        a[0] = h;
        a[1] = qx;
        a[2] = qy;
        if constexpr (NR == 4) a[3] = c;
        st_w<T, NR>(p0, k, a);
    } else {
        const T a[2] = {h, qx};
        T b[NR - 2];
        b[0] = qy;
        if constexpr (NR == 4) b[1] = c;
        st_w<T, 2>(p0, k, a);
        st_w<T, NR - 2>(p1, k, b);
    }
}

// Load a row of W^n for this lane.  CHECK: the row or the column may lie
// outside the domain (walls); such cells get benign placeholder values.
// `row` is the grid row.  The values are raw: a downward-marching tile
// negates qy where it uses them, not here, so that nothing waits on a load
// before its row is needed.  SM: streaming mode (non-temporal loads).
template <bool CHECK, bool SM, typename T, bool TR>
__device__ __forceinline__ void load_row(const CartArgs<T, TR> &A, int row, int col, bool colok, T &h,
                                         T &qx, T &qy, T &c, T &z, bool &rowok)
{
    rowok = true;
    if (row < 0 || row >= A.ny) {
        if (A.pery) row = row < 0 ? row + A.ny : row - A.ny;
        else rowok = false;
    }
    if (!CHECK || (rowok && colok)) {
        const uint32_t k = (uint32_t)row * (uint32_t)A.nx + (uint32_t)col;
        ld_rec<T, TR ? 4 : 3, SM>(A.in0, A.in1, k, h, qx, qy, c);
        z = at(A.z, k);
    } else {
        h = T(1);
        qx = qy = c = z = T(0);
    }
}

// Registers a wavefront carries from one row to the next.
template <typename T> struct Carry {
    PC<T> prev;                  // W^n of row r-1
    bool prevrow;                // row r-1 inside the domain (uniform)
    T ax_m, ax_x, ax_y, ax_c;    // x-edge fluctuation sums of row r-1
    T yb_m, yb_n, yb_t, yb_c;    // its bottom y-edge: mass, normal parts; transverse, pollutant fluxes
    T np_h, np_s, np_b;          // W^{n+1} of row r-2: h, sqrt(h), qy / sqrt(h)
    bool nprow;                  // row r-2 inside the domain
    T sx_prev, sybot_prev;       // Eq. (5) speed sums of row r-2 (x-edges, bottom edge)
    // recomputation variant only: W^n of row r-2 and W^{n+1} of row r-3
    PC<T> prev2;
    bool prev2row;
    T np2_h, np2_s, np2_b;
    bool np2row;
};

// A prefetched row of W^n for this lane.
template <typename T> struct Ld {
    T h, qx, qy, c, z;
    bool rowok;
};

// Per-tile constants.  A tile marches over "march rows" r = j0-2 ..
// j0+TY+1; an upward tile visits grid rows in that order (grid row = r), a
// downward tile in the opposite order (grid row = rbase - r) and works on
// the y-mirrored state (qy negated on load and store, walls and periodic
// wrap unchanged), so one code path serves both.  Rows rs0 .. rs1-1 (march
// numbering) are the tile's own rows that exist in the grid.
template <typename T> struct TileC {
    int i, col, j0, rlast, rs0, rs1, rbase;
    bool colok, xwall_lane, wlane;
    bool lwall_lane, prvok; // recomputation variant: a wall on the lane's left; column i-1 inside
    T fx, fy, g, lx, ly, g_half;
};

// Rows of W^n a wavefront keeps in flight ahead of the row it computes.
constexpr int PREFETCH = 2;

// One row step of a tile: row r of W^n arrives (cur), row r+PREFETCH is
// requested into nxt_ld, row r-1 of W^{n+1} is completed and stored, and
// the Eq. (5) speed sum of row r-2 is closed.  XW / YW: walls in x / y.
//
// RC: the recomputation variant.  Every cell evaluates all four of its
// edges itself -- the left x-edge and the bottom y-edge again, although the
// neighbouring lane and the previous row step already did -- instead of
// taking the neighbour's part of the shared edge (a DPP move, a carried
// register), for the fluxes and for the Eq. (5) speeds.  The inputs of a
// recomputed edge are bit-identical to the shared one's; the results agree
// to rounding (the compiler may contract the two evaluations' multiply-adds
// differently).
template <typename T, bool TR, bool XW, bool YW, bool DN, int FX, bool RC, bool SM>
__device__ __forceinline__ void row_step(const CartArgs<T, TR> &A, const TileC<T> &K, int r, const Carry<T> &I,
                                         Carry<T> &O, const Ld<T> &cur_ld, Ld<T> &nxt_ld, T &smax,
                                         uint64_t &bad_depth, uint64_t &bad_val)
{
    // the row PREFETCH ahead is requested before anything waits on row r
    if (r + PREFETCH <= K.rlast)
        load_row<XW || YW, SM>(A, DN ? K.rbase - (r + PREFETCH) : r + PREFETCH, K.col, K.colok, nxt_ld.h, nxt_ld.qx,
                           nxt_ld.qy, nxt_ld.c, nxt_ld.z, nxt_ld.rowok);
    const PC<T> cur = prep(cur_ld.h, cur_ld.qx, DN ? -cur_ld.qy : cur_ld.qy, cur_ld.c, cur_ld.z);
    const bool currow = cur_ld.rowok; // uniform across the wavefront
    const PC<T> &prev = I.prev;
    const T g = K.g, lx = K.lx, ly = K.ly;

    // ---- x-edge (lane, lane+1) of row r
    const T Rh = nxt(cur.h), Rs = nxt(cur.s), Ru = nxt(cur.u), Rv = nxt(cur.v), Rc = nxt(cur.cc),
            Rz = nxt(cur.z), Rq = nxt(cur.qx);
    EF<T> ex = flux<T, TR, FX>(cur.h, cur.s, cur.qx, cur.u, cur.v, cur.cc, cur.z, Rh, Rs, Rq, Ru, Rv, Rc, Rz, g);
    if (XW && K.xwall_lane) {
        ex.ft = ex.fc = T(0);
        if (K.colok) { // wall on the right of this lane's cell
            wall(cur.h, cur.qx, g, ex.am, ex.an);
            ex.bm = ex.bn = T(0);
        } else { // wall on the left of the next lane's cell: qn = -qx;
                 // back-rotation of the normal momentum n -> -n
            T m, n;
            wall(Rh, -Rq, g, m, n);
            ex.am = ex.an = T(0);
            ex.bm = m;
            ex.bn = -n;
        }
    }
    if constexpr (RC) {
        // the left x-edge (lane-1, lane) of row r, evaluated again here
        const T Lh = prv(cur.h), Ls = prv(cur.s), Lu = prv(cur.u), Lv = prv(cur.v), Lc = prv(cur.cc),
                Lz = prv(cur.z), Lq = prv(cur.qx);
        EF<T> el = flux<T, TR, FX>(Lh, Ls, Lq, Lu, Lv, Lc, Lz, cur.h, cur.s, cur.qx, cur.u, cur.v, cur.cc, cur.z, g);
        if (XW && K.lwall_lane) {
            el.bm = el.bn = el.ft = el.fc = T(0);
            if (K.colok) { // wall on the left of this lane's cell (as seen by the lane on the left)
                T m, n;
                wall(cur.h, -cur.qx, g, m, n);
                el.bm = m;
                el.bn = -n;
            }
        }
        O.ax_m = ex.am + el.bm;
        O.ax_x = ex.an + el.bn;
        O.ax_y = ex.ft - el.ft;
        O.ax_c = TR ? ex.fc - el.fc : T(0);
    } else {
        O.ax_m = ex.am + prv(ex.bm);
        O.ax_x = ex.an + prv(ex.bn);
        O.ax_y = ex.ft - prv(ex.ft);
        O.ax_c = TR ? ex.fc - prv(ex.fc) : T(0);
    }

    // ---- y-edge (row r-1, row r): normal (0, 1), qn = qy, ut = -u;
    // back-rotation (m, n, t, c) -> (m, -t, n, c)
    EF<T> ey = flux<T, TR, FX>(prev.h, prev.s, prev.qy, prev.v, -prev.u, prev.cc, prev.z, cur.h, cur.s, cur.qy, cur.v,
                           -cur.u, cur.cc, cur.z, g);
    if (YW && I.prevrow != currow) {
        ey.ft = ey.fc = T(0);
        if (I.prevrow) { // wall above row r-1
            wall(prev.h, prev.qy, g, ey.am, ey.an);
            ey.bm = ey.bn = T(0);
        } else { // wall below row r: normal (0, -1), qn = -qy; the normal
                 // momentum maps back as n -> -n
            T m, n;
            wall(cur.h, -cur.qy, g, m, n);
            ey.am = ey.an = T(0);
            ey.bm = m;
            ey.bn = -n;
        }
    }

    O.np_h = I.np_h;
    O.np_s = I.np_s;
    O.np_b = I.np_b;
    O.nprow = I.nprow;
    O.sx_prev = I.sx_prev;
    O.sybot_prev = I.sybot_prev;
    if constexpr (RC) {
        O.np2_h = I.np2_h;
        O.np2_s = I.np2_s;
        O.np2_b = I.np2_b;
        O.np2row = I.np2row;
    }
    if (r >= K.j0) {
        // ---- complete row r-1: W^{n+1} = W^n - dt/|V| sum |G| fluct, the
        // x- and y-edge sums scaled by dt |G_x| / |V| and dt |G_y| / |V|;
        // y-edge parts map back as (m, n, t, c) -> (m, -t, n, c) (the edge
        // frame's transverse axis is -x); the transverse and pollutant rows
        // are flux differences (top minus bottom, right minus left)
        T ybm = I.yb_m, ybt = I.yb_t, ybn = I.yb_n, ybc = I.yb_c;
        if constexpr (RC) { // the bottom y-edge (r-2, r-1), evaluated again
            const PC<T> &p2 = I.prev2;
            EF<T> eb = flux<T, TR, FX>(p2.h, p2.s, p2.qy, p2.v, -p2.u, p2.cc, p2.z, prev.h, prev.s, prev.qy, prev.v,
                                       -prev.u, prev.cc, prev.z, g);
            if (YW && I.prev2row != I.prevrow) {
                eb.bm = eb.bn = eb.ft = eb.fc = T(0);
                if (I.prevrow) { // wall below row r-1
                    T m, n;
                    wall(prev.h, -prev.qy, g, m, n);
                    eb.bm = m;
                    eb.bn = -n;
                }
            }
            ybm = eb.bm;
            ybt = eb.ft;
            ybn = eb.bn;
            ybc = eb.fc;
        }
        const T ym = ybm + ey.am;
        const T yt = ey.ft - ybt;
        const T yn = ybn + ey.an;
        const T yc = ey.fc - ybc;
        const T fx = K.fx, fy = K.fy;
        const T h1 = prev.h - fx * I.ax_m - fy * ym;
        const T qx1 = prev.qx - fx * I.ax_x + fy * yt;
        const T qy1 = prev.qy - fx * I.ax_y - fy * yn;
        const T c1 = TR ? prev.c - fx * I.ax_c - fy * yc : T(0);
        // ---- Eq. (5) speeds of W^{n+1}
        const T rq = FM<T>::rsq(h1);
        const T s1 = h1 * rq, a1 = qx1 * rq, b1 = qy1 * rq;
        const T Nh = nxt(h1), Ns = nxt(s1), Na = nxt(a1);
        T exs = espeed(h1, s1, a1, Nh, Ns, Na, g);
        if (XW && K.xwall_lane) exs = FM<T>::sqrt(g * (K.colok ? h1 : Nh));
        T exl;
        if constexpr (RC) { // the left x-edge's speed, evaluated again
            const T Ph = prv(h1), Ps = prv(s1), Pa = prv(a1);
            exl = espeed(Ph, Ps, Pa, h1, s1, a1, g);
            if (XW && K.lwall_lane) exl = FM<T>::sqrt(g * (K.prvok ? Ph : h1));
        } else {
            exl = prv(exs);
        }
        const T sx_cur = lx * (exs + exl);
        if (r >= K.j0 + 1) {
            // y-edge (r-2, r-1) of W^{n+1} completes the speed sum of row r-2
            T eys;
            if (!YW || (I.nprow && I.prevrow)) eys = espeed(I.np_h, I.np_s, I.np_b, h1, s1, b1, g);
            else eys = FM<T>::sqrt(g * (I.nprow ? I.np_h : h1));
            eys *= ly;
            T ysb = I.sybot_prev;
            if constexpr (RC) { // row r-2's bottom edge (r-3, r-2), evaluated again
                if (!YW || (I.np2row && I.nprow)) ysb = espeed(I.np2_h, I.np2_s, I.np2_b, I.np_h, I.np_s, I.np_b, g);
                else ysb = FM<T>::sqrt(g * (I.np2row ? I.np2_h : I.np_h));
                ysb *= ly;
            }
            const int rr = r - 2;
            if (rr >= K.rs0 && rr < K.rs1 && K.wlane) smax = fmax(smax, I.sx_prev + ysb + eys);
            O.sybot_prev = eys;
        }
        // ---- store row r-1 of the tile
        const int wr = r - 1;
        if (wr >= K.rs0 && wr < K.rs1 && K.wlane) {
            const uint32_t k = (uint32_t)(DN ? K.rbase - wr : wr) * (uint32_t)A.nx + (uint32_t)K.i;
            st_rec<T, TR ? 4 : 3>(A.out0, A.out1, k, h1, qx1, DN ? -qy1 : qy1, c1);
            // lane masks of the wavefront (scalar registers, no per-lane select)
            bad_depth |= __ballot(!(h1 > T(0)));
            bad_val |= __ballot(!isfinite(h1 + qx1 + qy1 + c1));
        }
        if constexpr (RC) {
            O.np2_h = I.np_h;
            O.np2_s = I.np_s;
            O.np2_b = I.np_b;
            O.np2row = I.nprow;
        }
        O.np_h = h1;
        O.np_s = s1;
        O.np_b = b1;
        O.nprow = I.prevrow;
        O.sx_prev = sx_cur;
    }
    // bottom part of the y-edge for row r (edge frame)
    O.yb_m = ey.bm;
    O.yb_t = ey.ft;
    O.yb_n = ey.bn;
    O.yb_c = ey.fc;
    if constexpr (RC) {
        O.prev2 = I.prev;
        O.prev2row = I.prevrow;
    }
    O.prev = cur;
    O.prevrow = currow;
}

// One wavefront's tile.  XW: the tile has a wall among its x-edges; YW: the
// tile's rows reach a wall in y.  Tiles with neither (almost all of them)
// run without any wall code.  Returns the tile's largest Eq. (5) speed sum
// sum |G| ||D|| (the smallest dt candidate is 2 gamma |V| over it).
template <typename T, bool TR, bool XW, bool YW, bool DN, int FX, bool RC, bool SM>
__device__ __forceinline__ void cart_tile(const CartArgs<T, TR> &A, int tile, int lane, double dtd, T &smax_out,
                                          unsigned &bad_out)
{
    const int strip = tile % A.nstrips, rb = tile / A.nstrips;
    TileC<T> K;
    K.i = strip * CART_COLS - 2 + lane; // column of this lane
    K.j0 = rb * A.ty;
    auto wrapc = [&](int c, bool &ok) {
        ok = true;
        if (c < 0 || c >= A.nx) {
            if (A.perx) c = ((c % A.nx) + A.nx) % A.nx;
            else ok = false;
        }
        return c;
    };
    bool nxtok;
    K.col = wrapc(K.i, K.colok);
    (void)wrapc(K.i + 1, nxtok);
    // lanes whose x-edge to the right is a wall (either side outside)
    K.xwall_lane = K.colok != nxtok;
    (void)wrapc(K.i - 1, K.prvok);
    K.lwall_lane = K.colok != K.prvok;
    K.wlane = lane >= 2 && lane < 2 + CART_COLS && K.i >= 0 && K.i < A.nx;
    K.rlast = K.j0 + A.ty + 1; // last row loaded
    K.rbase = 2 * K.j0 + A.ty - 1; // DN: grid row = rbase - march row
    const int jtop = min(K.j0 + A.ty, A.ny);
    K.rs0 = DN ? K.rbase - jtop + 1 : K.j0;
    K.rs1 = DN ? K.j0 + A.ty : jtop;
    K.fx = (T)(dtd / (double)A.dx); // dt |G_x| / |V|, |G_x| = dy
    K.fy = (T)(dtd / (double)A.dy); // dt |G_y| / |V|, |G_y| = dx
    K.g = A.g;
    K.lx = A.dy; // length of an x-edge
    K.ly = A.dx; // length of a y-edge

    T smax = T(0);
    uint64_t bad_depth = 0, bad_val = 0;
    Carry<T> c0, c1;
    Ld<T> l0, l1, l2, l3;
    {
        Ld<T> p;
        load_row<XW || YW, SM>(A, DN ? K.rbase - (K.j0 - 2) : K.j0 - 2, K.col, K.colok, p.h, p.qx, p.qy, p.c, p.z, p.rowok);
        c0.prevrow = p.rowok;
        c0.ax_m = c0.ax_x = c0.ax_y = c0.ax_c = T(0);
        c0.yb_m = c0.yb_n = c0.yb_t = c0.yb_c = T(0);
        c0.np_h = T(1);
        c0.np_s = T(1);
        c0.np_b = T(0);
        c0.nprow = false;
        c0.sx_prev = c0.sybot_prev = T(0);
        c0.prev2row = false;
        c0.np2_h = T(1);
        c0.np2_s = T(1);
        c0.np2_b = T(0);
        c0.np2row = false;
        load_row<XW || YW, SM>(A, DN ? K.rbase - (K.j0 - 1) : K.j0 - 1, K.col, K.colok, l0.h, l0.qx, l0.qy, l0.c, l0.z, l0.rowok);
        load_row<XW || YW, SM>(A, DN ? K.rbase - K.j0 : K.j0, K.col, K.colok, l1.h, l1.qx, l1.qy, l1.c, l1.z, l1.rowok);
        c0.prev = prep(p.h, p.qx, DN ? -p.qy : p.qy, p.c, p.z);
        c0.prev2 = c0.prev;
    }
    // Four rows per trip: the carried registers alternate between c0 and c1
    // and the four row buffers rotate (row r in one, row r+2 requested into
    // another), so no register is copied between rows.
    int r = K.j0 - 1;
    for (; r + 3 <= K.rlast; r += 4) {
        row_step<T, TR, XW, YW, DN, FX, RC, SM>(A, K, r, c0, c1, l0, l2, smax, bad_depth, bad_val);
        row_step<T, TR, XW, YW, DN, FX, RC, SM>(A, K, r + 1, c1, c0, l1, l3, smax, bad_depth, bad_val);
        row_step<T, TR, XW, YW, DN, FX, RC, SM>(A, K, r + 2, c0, c1, l2, l0, smax, bad_depth, bad_val);
        row_step<T, TR, XW, YW, DN, FX, RC, SM>(A, K, r + 3, c1, c0, l3, l1, smax, bad_depth, bad_val);
    }
    if (r <= K.rlast) row_step<T, TR, XW, YW, DN, FX, RC, SM>(A, K, r, c0, c1, l0, l2, smax, bad_depth, bad_val);
    if (r + 1 <= K.rlast) row_step<T, TR, XW, YW, DN, FX, RC, SM>(A, K, r + 1, c1, c0, l1, l3, smax, bad_depth, bad_val);
    if (r + 2 <= K.rlast) row_step<T, TR, XW, YW, DN, FX, RC, SM>(A, K, r + 2, c0, c1, l2, l0, smax, bad_depth, bad_val);
    smax_out = smax;
    bad_out = (bad_depth ? FLAG_DEPTH : 0u) | (bad_val ? FLAG_NONFINITE : 0u);
}

// The tile variant for its walls (x, y) and march direction.
template <typename T, bool TR, bool DN, int FX, bool RC, bool SM>
__device__ __forceinline__ void cart_tile_dispatch(const CartArgs<T, TR> &A, int tile, int lane, double dtd, bool xw,
                                                   bool yw, T &smax, unsigned &bad)
{
    if (!xw && !yw) cart_tile<T, TR, false, false, DN, FX, RC, SM>(A, tile, lane, dtd, smax, bad);
    else if (!yw) cart_tile<T, TR, true, false, DN, FX, RC, SM>(A, tile, lane, dtd, smax, bad);
    else if (!xw) cart_tile<T, TR, false, true, DN, FX, RC, SM>(A, tile, lane, dtd, smax, bad);
    else cart_tile<T, TR, true, true, DN, FX, RC, SM>(A, tile, lane, dtd, smax, bad);
}

template <typename T, bool TR, int FX = FLUX_IR, bool RC = false, bool SM = false>
__global__ __launch_bounds__(64) void k_cart_fused(CartArgs<T, TR> A)
{
    const int lane = threadIdx.x;
    // XCD-aware tile index: workgroup w runs on XCD w % 8.  A reversed step
    // starts with the tiles that the step before it wrote last.
    const int w = blockIdx.x;
    const int tile0 = (w % NUM_XCD) * A.per_xcd + w / NUM_XCD;
    const int tile = A.rev ? A.per_xcd * NUM_XCD - 1 - tile0 : tile0;

    // dt^n from the partial minima of the previous launch
    const int bank = (int)((A.step + A.bank0) % 3);
    double dtd = A.part[bank * NPART + lane];
    dtd = wave_min(dtd);
    if (w == 0) {
        A.part[((bank + 2) % 3) * NPART + lane] = __builtin_inf();
        if (lane == 0) {
            A.book.hist[A.step] = dtd;
            A.book.last[0] = dtd;
            A.book.t[0] += dtd;
        }
    }
    if (tile >= A.ntiles) return;

    const int strip = tile % A.nstrips, rb = tile / A.nstrips;
    const int i0 = strip * CART_COLS - 2, j0 = rb * A.ty;
    const bool xw = !A.perx && (i0 < 0 || i0 + CART_LANES > A.nx);
    const bool yw = !A.pery && (j0 - 2 < 0 || j0 + A.ty + 1 >= A.ny);
    T smax;
    unsigned bad;
    // on large grids odd row blocks march downward: neighbouring blocks then
    // reach the rows they share (each other's halo) at about the same time,
    // while those rows are still in L2
    if (A.alt && (rb & 1)) cart_tile_dispatch<T, TR, true, FX, RC, SM>(A, tile, lane, dtd, xw, yw, smax, bad);
    else cart_tile_dispatch<T, TR, false, FX, RC, SM>(A, tile, lane, dtd, xw, yw, smax, bad);

    // the tile's dt candidate 2 gamma |V| / max sum |G| ||D|| (Eq. (5))
    const double dmin = wave_min(smax > T(0) ? (double)(T(2) * A.cfl * A.dx * A.dy / smax) : __builtin_inf());
    if (lane == 0 && dmin >= 0.0 && dmin < __builtin_inf())
        atomicMin(reinterpret_cast<unsigned long long *>(A.part + ((bank + 1) % 3) * NPART + (w % NPART)),
                  (unsigned long long)__double_as_longlong(dmin));
    if (bad) atomicOr(A.book.flags, bad);
}

// dt of the initial state (Eq. (5) on W^0), in the first batch after a new
// state or a cfl change: one wavefront per tile of DT0_COLS columns (lanes
// 1..DT0_COLS; lanes 0 and 63 are the halo columns) by DT0_ROWS rows,
// marching up its rows like the fused kernel: a row of each field is one
// coalesced load, the x-neighbour is the next lane and the y-neighbour the
// previous row in registers.  Each edge speed is evaluated once, with the
// arithmetic the fused kernel applies to W^{n+1} (espeed, and sqrt(g h) at a
// wall), so every step's dt comes from the same formula.  Four wavefronts
// per workgroup, one atomic min per workgroup into bank 0.
constexpr int DT0_COLS = 62;
constexpr int DT0_ROWS = 16;
constexpr int DT0_WAVES = 4;

struct Dt0Args {
    const void *rec0, *rec1; // W^0, the record planes
    int nx, ny, perx, pery;
    double dx, dy, g, cfl;
    int nstrips, ntiles;
    double *part;
};

// CHECK: the tile's rows or columns reach beyond the grid (wrap or wall).
template <typename T, int NR, bool CHECK>
__device__ __forceinline__ T dt0_tile(const Dt0Args &A, int tile, int lane)
{
    const T *W0 = (const T *)A.rec0, *W1 = (const T *)A.rec1;
    const int strip = tile % A.nstrips, rb = tile / A.nstrips;
    const int i = strip * DT0_COLS - 1 + lane;
    const int j0 = rb * DT0_ROWS, jend = min(j0 + DT0_ROWS, A.ny);
    // index inside the grid (periodic) or flagged outside (wall); a tile's
    // columns may pass a narrow periodic grid more than once
    auto wrap = [](int c, int n, int per, bool &ok) {
        ok = true;
        if (c < 0 || c >= n) {
            if (per) c = ((c % n) + n) % n;
            else ok = false;
        }
        return c;
    };
    bool colok = true, nxtok = true;
    int col = i;
    if (CHECK) {
        col = wrap(i, A.nx, A.perx, colok);
        (void)wrap(i + 1, A.nx, A.perx, nxtok);
    }
    const bool xwall_lane = colok != nxtok; // the lane's right edge is a wall
    const bool wlane = lane >= 1 && lane <= DT0_COLS && i < A.nx;
    const T g = (T)A.g, lx = (T)A.dy, ly = (T)A.dx;

    // a row of h, qx, qy for this lane (placeholders outside a wall)
    struct Row {
        T h, qx, qy;
        bool ok;
    };
    auto load = [&](int r) {
        Row w;
        w.ok = true;
        int row = r;
        if (CHECK) row = wrap(r, A.ny, A.pery, w.ok);
        w.h = T(1);
        w.qx = w.qy = T(0);
        if (!CHECK || (w.ok && colok)) {
            const uint32_t k = (uint32_t)row * (uint32_t)A.nx + (uint32_t)col;
            T c;
            ld_rec<T, NR>(W0, W1, k, w.h, w.qx, w.qy, c);
        }
        return w;
    };

    T smax = T(0);
    T ph = T(1), ps = T(1), pb = T(0), psx = T(0), pyb = T(0);
    bool prow = false;
    // row r of the march (j0-1 .. jend): speeds of its x-edges, the y-edge
    // below it, and the closed speed sum of row r-1
    auto step = [&](const Row &w, int r) {
        const T h = w.h, qx = w.qx, qy = w.qy;
        const T rq = FM<T>::rsq(h);
        const T s = h * rq, a = qx * rq, b = qy * rq;
        const T Nh = nxt(h), Ns = nxt(s), Na = nxt(a);
        T exs = espeed(h, s, a, Nh, Ns, Na, g);
        if (CHECK && xwall_lane) exs = FM<T>::sqrt(g * (colok ? h : Nh));
        const T sx = lx * (exs + prv(exs));
        if (r >= j0) {
            // the y-edge (r-1, r): row r-1's top edge and row r's bottom edge
            T eys;
            if (!CHECK || (prow && w.ok)) eys = espeed(ph, ps, pb, h, s, b, g);
            else eys = FM<T>::sqrt(g * (prow ? ph : h));
            eys *= ly;
            if (r - 1 >= j0 && wlane) smax = fmax(smax, psx + pyb + eys);
            pyb = eys;
        }
        ph = h;
        ps = s;
        pb = b;
        psx = sx;
        prow = w.ok;
    };
    // every row of the march (j0-1 .. j0+DT0_ROWS) is requested before the
    // first is used: a short tile's loads are all in flight at once
    Row w[DT0_ROWS + 2];
#pragma unroll
    for (int k = 0; k < DT0_ROWS + 2; ++k) w[k] = load(min(j0 - 1 + k, jend));
#pragma unroll
    for (int k = 0; k < DT0_ROWS + 2; ++k)
        if (j0 - 1 + k <= jend) step(w[k], j0 - 1 + k);
    return smax;
}

template <typename T, int NR> __global__ __launch_bounds__(64 * DT0_WAVES) void k_cart_dt0(Dt0Args A)
{
    const int lane = threadIdx.x & 63;
    const int tile = blockIdx.x * DT0_WAVES + (threadIdx.x >> 6);
    T smax = T(0);
    if (tile < A.ntiles) { // uniform over the wavefront
        const int strip = tile % A.nstrips, rb = tile / A.nstrips;
        const int i0 = strip * DT0_COLS - 1, j0 = rb * DT0_ROWS;
        const bool edge = i0 < 0 || i0 + 64 > A.nx || j0 - 1 < 0 || j0 + DT0_ROWS + 1 > A.ny;
        smax = edge ? dt0_tile<T, NR, true>(A, tile, lane) : dt0_tile<T, NR, false>(A, tile, lane);
    }
    const T two_cfl_area = T(2) * (T)A.cfl * (T)A.dx * (T)A.dy;
    const double cand = smax > T(0) ? (double)(two_cfl_area / smax) : __builtin_inf();
    block_min_to_slot(cand, A.part + (blockIdx.x % NPART));
}

// Launch of the streaming-mode kernel for one step.  Its instantiations are
// compiled in a translation unit of their own (this file built a second time
// with SWE_CART_STREAM_TU defined), in parallel with the rest of the file.
template <typename T, bool TR, int FX, bool RC>
void launch_cart_stream(unsigned grid, hipStream_t s, const CartArgs<T, TR> &A);

#ifdef SWE_CART_STREAM_TU

template <typename T, bool TR, int FX, bool RC>
void launch_cart_stream(unsigned grid, hipStream_t s, const CartArgs<T, TR> &A)
{
    hipLaunchKernelGGL((k_cart_fused<T, TR, FX, RC, true>), dim3(grid), dim3(CART_LANES), 0, s, A);
}

// every flux and path that launch_cart_batch dispatches
#define SWE_CART_STREAM_INST(T, TR)                                                                          \
    template void launch_cart_stream<T, TR, FLUX_IR, false>(unsigned, hipStream_t, const CartArgs<T, TR> &);   \
    template void launch_cart_stream<T, TR, FLUX_IR_HH, false>(unsigned, hipStream_t, const CartArgs<T, TR> &); \
    template void launch_cart_stream<T, TR, FLUX_ROE, false>(unsigned, hipStream_t, const CartArgs<T, TR> &);  \
    template void launch_cart_stream<T, TR, FLUX_ROE_HH, false>(unsigned, hipStream_t, const CartArgs<T, TR> &); \
    template void launch_cart_stream<T, TR, FLUX_IR, true>(unsigned, hipStream_t, const CartArgs<T, TR> &);
SWE_CART_STREAM_INST(float, false)
SWE_CART_STREAM_INST(float, true)
SWE_CART_STREAM_INST(double, false)
SWE_CART_STREAM_INST(double, true)
#undef SWE_CART_STREAM_INST

#else // the rest of the path

// Batch start: elapsed time and error flags to zero; the partial minima
// too when the batch starts from a fresh state (else the previous batch's
// last launch left dt of the current state in bank bank0).
__global__ void k_cart_init(double *part, StepBook book, int reset_part)
{
    const int t = threadIdx.x;
    if (reset_part)
        for (int k = t; k < 3 * NPART; k += blockDim.x) part[k] = __builtin_inf();
    if (t == 0) {
        book.t[0] = 0.0;
        book.flags[0] = 0u;
    }
}

template <typename T, bool TR> static CartArgs<T, TR> cart_args(swe_ctx *c, int64_t step, double cfl)
{
    CartArgs<T, TR> A;
    const int in = c->cur ^ (int)(step & 1), out = in ^ 1;
    A.in0 = (const T *)c->state[in];
    A.in1 = A.in0 + cart_plane1(c);
    A.out0 = (T *)c->state[out];
    A.out1 = A.out0 + cart_plane1(c);
    A.z = (const T *)c->zbed;
    A.nx = (int)c->nx;
    A.ny = (int)c->ny;
    A.perx = c->bc_x == SWE_BC_PERIODIC;
    A.pery = c->bc_y == SWE_BC_PERIODIC;
    A.dx = (T)c->dx;
    A.dy = (T)c->dy;
    A.g = (T)c->g;
    A.cfl = (T)cfl;
    A.ty = c->cart_ty;
    A.alt = c->cart_alt;
    A.rev = c->cart_stream ? in : 0;
    A.nstrips = (int)((c->nx + CART_COLS - 1) / CART_COLS);
    const int nrb = (int)((c->ny + A.ty - 1) / A.ty);
    A.ntiles = A.nstrips * nrb;
    A.per_xcd = (A.ntiles + NUM_XCD - 1) / NUM_XCD;
    A.part = c->cart_part;
    A.book = c->book;
    A.step = step;
    A.bank0 = c->bank0;
    return A;
}

template <typename T, bool TR, int FX = FLUX_IR, bool RC = false>
static hipError_t cart_batch_t(swe_ctx *c, int32_t nsteps, double cfl)
{
    // dt of the current state: left by the previous batch (same state, same
    // cfl), else computed here into bank 0
    const bool fresh = !c->dt_ready || c->dt_cfl != cfl;
    if (fresh) c->bank0 = 0;
    hipLaunchKernelGGL(k_cart_init, dim3(1), dim3(64), 0, c->stream, c->cart_part, c->book, fresh ? 1 : 0);
    if (fresh) {
        Dt0Args D;
        D.rec0 = c->state[c->cur];
        D.rec1 = (const T *)c->state[c->cur] + cart_plane1(c);
        D.nx = (int)c->nx;
        D.ny = (int)c->ny;
        D.perx = c->bc_x == SWE_BC_PERIODIC;
        D.pery = c->bc_y == SWE_BC_PERIODIC;
        D.dx = c->dx;
        D.dy = c->dy;
        D.g = c->g;
        D.cfl = cfl;
        D.nstrips = (int)((c->nx + DT0_COLS - 1) / DT0_COLS);
        D.ntiles = D.nstrips * (int)((c->ny + DT0_ROWS - 1) / DT0_ROWS);
        D.part = c->cart_part; // bank 0
        const unsigned nb0 = (unsigned)((D.ntiles + DT0_WAVES - 1) / DT0_WAVES);
        hipLaunchKernelGGL((k_cart_dt0<T, TR ? 4 : 3>), dim3(nb0), dim3(64 * DT0_WAVES), 0, c->stream, D);
    }
    for (int64_t s = 0; s < nsteps; ++s) {
        const CartArgs<T, TR> A = cart_args<T, TR>(c, s, cfl);
        const unsigned grid = (unsigned)(A.per_xcd * NUM_XCD);
        if (c->cart_stream)
            launch_cart_stream<T, TR, FX, RC>(grid, c->stream, A);
        else
            hipLaunchKernelGGL((k_cart_fused<T, TR, FX, RC>), dim3(grid), dim3(CART_LANES), 0, c->stream, A);
    }
    return hipGetLastError();
}

template <int FX, bool RC> static hipError_t cart_batch_fx(swe_ctx *c, int32_t nsteps, double cfl)
{
    const bool f32 = c->prec == SWE_F32;
    if (c->ntracers)
        return f32 ? cart_batch_t<float, true, FX, RC>(c, nsteps, cfl) : cart_batch_t<double, true, FX, RC>(c, nsteps, cfl);
    return f32 ? cart_batch_t<float, false, FX, RC>(c, nsteps, cfl) : cart_batch_t<double, false, FX, RC>(c, nsteps, cfl);
}

// The caller's separate arrays (one per variable) <-> the record planes of
// the structured path, for the device-memory set and get calls.
template <typename T, int NR>
__global__ void k_cart_pack(const T *__restrict__ a0, const T *__restrict__ a1, const T *__restrict__ a2,
                            const T *__restrict__ a3, T *__restrict__ p0, T *__restrict__ p1, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    st_rec<T, NR>(p0, p1, (uint32_t)i, a0[i], a1[i], a2[i], NR == 4 ? a3[i] : T(0));
}
template <typename T, int NR>
__global__ void k_cart_unpack(const T *__restrict__ p0, const T *__restrict__ p1, T *__restrict__ a0,
                              T *__restrict__ a1, T *__restrict__ a2, T *__restrict__ a3, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    T h, qx, qy, c;
    ld_rec<T, NR>(p0, p1, (uint32_t)i, h, qx, qy, c);
    a0[i] = h;
    a1[i] = qx;
    a2[i] = qy;
    if (NR == 4) a3[i] = c;
}

template <typename T, int NR> static hipError_t cart_pack_t(swe_ctx *c, const void *const *soa, void *rec, int pack)
{
    const unsigned nb = (unsigned)((c->N + 255) / 256);
    T *v[4];
    for (int k = 0; k < 4; ++k) v[k] = k < NR ? (T *)soa[k] : nullptr;
    T *p0 = (T *)rec, *p1 = p0 + cart_plane1(c);
    if (pack)
        hipLaunchKernelGGL((k_cart_pack<T, NR>), dim3(nb), dim3(256), 0, c->stream, v[0], v[1], v[2], v[3], p0, p1,
                           c->N);
    else
        hipLaunchKernelGGL((k_cart_unpack<T, NR>), dim3(nb), dim3(256), 0, c->stream, p0, p1, v[0], v[1], v[2],
                           v[3], c->N);
    return hipGetLastError();
}

hipError_t launch_cart_pack(swe_ctx *c, const void *const *soa, void *rec, int pack)
{
    if (c->prec == SWE_F32) return c->nv == 4 ? cart_pack_t<float, 4>(c, soa, rec, pack) : cart_pack_t<float, 3>(c, soa, rec, pack);
    return c->nv == 4 ? cart_pack_t<double, 4>(c, soa, rec, pack) : cart_pack_t<double, 3>(c, soa, rec, pack);
}

hipError_t launch_cart_batch(swe_ctx *c, int32_t nsteps, double cfl)
{
    if (c->path == SWE_PATH_RECOMPUTE) return cart_batch_fx<FLUX_IR, true>(c, nsteps, cfl); // IR-Roe only
    if (c->classical) return c->hh ? cart_batch_fx<FLUX_ROE_HH, false>(c, nsteps, cfl)
                                   : cart_batch_fx<FLUX_ROE, false>(c, nsteps, cfl);
    if (c->hh) return cart_batch_fx<FLUX_IR_HH, false>(c, nsteps, cfl);
    return cart_batch_fx<FLUX_IR, false>(c, nsteps, cfl);
}

#endif // SWE_CART_STREAM_TU

} // namespace swe
