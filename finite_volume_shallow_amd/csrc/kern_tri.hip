// Fused triangle-mesh path: one kernel launch per time step.
//
// The mesh is cut into blocks of B consecutive cells of a Morton order (the
// library sorts the cells by the Morton code of their centroids, so a block
// is a compact patch).  The launch for step n gives each block one
// workgroup, which
//   1. loads W^n and the bed of its cells plus two rings of neighbours into
//      LDS (block cells are one coalesced range, the rings a gather list),
//   2. evaluates every edge touching the block or ring 1 once ([IR] Sec. 2.2
//      steps 1-4: rotate to the edge frame, Roe fluctuations with the
//      path-conservative bed term, upwinded transverse momentum and [MG]
//      pollutant, rotate back) and parks |G| T^-1 (fluctuation) of both
//      sides in per-edge LDS slots,
//   3. updates the block and ring 1 (Eq. (4) with dt^n): each cell gathers
//      its three edge slots in a fixed order -- no atomics, deterministic,
//   4. evaluates the Eq. (5) wave speeds of W^{n+1} on the block's edges
//      (both sides of those edges are now in LDS), forms each block cell's
//      2 gamma |V| / sum |G| ||D|| and folds the block minimum into the
//      partial minima the next launch reduces to dt^{n+1},
//   5. writes W^{n+1} of the block (ping-pong buffers).
// Ring-1 cells are updated redundantly by the neighbouring blocks that need
// them; that is what lets one launch read and write the state once.
//
// Workgroups are mapped XCD-aware: workgroup w runs on XCD w % 8 and the
// blocks are dealt to the XCDs in contiguous bands, so neighbouring patches
// (which share halo cells) share an L2.
#include "dt_reduce.hpp"
#include "roe_device.hpp"
#include "swe_internal.hpp"

namespace swe {

constexpr int TRI_XCD = 8;
constexpr int TRI_NPART = 64;
constexpr int TRI_CTR_STRIDE = 64; // 32-bit words from one block counter to the next: 256 bytes
static_assert(3 * TRI_NPART + 3 * TRI_XCD * TRI_CTR_STRIDE / 2 <= PART_DOUBLES, "partial minima and block counters");

template <typename T> struct TriArgs {
    const T *in;  // W^n: one record of the NV conserved variables per cell
    T *out;       // W^{n+1}, records as `in`
    const T *z;
    int64_t N;
    int B, nblocks, per_xcd, lc_max, e_max;
    const int32_t *halo_off, *halo_ids, *n1, *edge_off, *e_s0, *slot_off;
    const uint32_t *e_ab;
    const T *e_gx, *e_gy; // |G| eta of the local edges
    const uint16_t *slots;
    const uint32_t *slots32; // the pipelined kernel's 4-byte rows (three 10-bit record indices)
    const T *iarea;
    T g, r, cfl;
    double *part;
    unsigned *ctr; // [3][TRI_XCD] block counters of the pipelined kernel (bank of the launch, per XCD band),
                   // TRI_CTR_STRIDE words apart
    int rev;       // the pipelined kernel walks its bands backwards (every other step)
    StepBook book;
    int64_t step;  // index of the step within the batch (dt history)
    int bank0;     // partial-minimum bank of the batch's first step
};

// Largest |eigenvalue| of the two-layer Roe matrix (the outer roots of the
// quartic, see roe_device.hpp), edge-frame states L, R with their per-cell
// sqrt(h_k), 1/h_k in pL, pR.
template <typename T>
__device__ __forceinline__ T roe2_speed(const T *L, const T *pL, const T *R, const T *pR, T g, T r, bool &nonhyp)
{
    const T u1 = (L[1] * pL[1] * pL[0] + R[1] * pR[1] * pR[0]) * FM<T>::rcp(pL[0] + pR[0]);
    const T u2 = (L[4] * pL[3] * pL[2] + R[4] * pR[3] * pR[2]) * FM<T>::rcp(pL[2] + pR[2]);
    const T c1 = g * T(0.5) * (L[0] + R[0]);
    const T c2 = g * T(0.5) * (L[3] + R[3]);
    const T rc = r * c1 * c2;
    const T m = T(0.5) * (u1 + u2), d1 = u1 - m, d2 = u2 - m;
    T hi, lo;
    outer_roots(d1, d2, c1, c2, rc, hi, lo);
    // inner pair real?  (deflated quadratic discriminant)
    const T p1 = d1 * d1 - c1, p2 = d2 * d2 - c2;
    const T a3 = T(-2) * (d1 + d2), a2 = p1 + p2 + T(4) * d1 * d2;
    const T b1 = a3 + (hi + lo), b0 = a2 + (hi + lo) * b1 - hi * lo;
    if (b1 * b1 - T(4) * b0 < T(0)) nonhyp = true;
    return fmax(fabs(hi + m), fabs(lo + m));
}

// LDS records.  A wavefront's 8-byte LDS read is served in two halves of
// 32 lanes, each taking as many cycles as the largest number of distinct
// addresses in one 8-byte bank slot ((address / 8) mod 32): lanes reading
// consecutive records of an odd number of 8-byte reals meet no conflict, so
// every record stride here is odd (in reals); field offsets are constants.
//   cell: the NV conserved variables, z and (one layer) sqrt(h) and 1/h in
//   one record of SA reals, so that an edge's gather of a cell takes the
//   fewest LDS instructions;
//   edge fluctuations: side a of every edge, then side b, ER reals each.
template <int NL, int NV> struct TriRec {
    static constexpr int SA = NL == 1 ? ((NV + 3) | 1) : ((NV + 1) | 1);
    static constexpr int AX = 0; // no separate per-cell record
    static constexpr int ER = NV | 1;
};

// View of local cell l: its record (state, z and, one layer, sqrt(h), 1/h).
template <typename T, int NL, int NV> struct TriCell {
    T *s;
    __device__ __forceinline__ TriCell(T *sm, int lcm, int l) : s(sm + l * TriRec<NL, NV>::SA) {}
    __device__ __forceinline__ T &z() const { return s[NV]; }
    __device__ __forceinline__ T &sq() const { return s[NV + 1]; } // sqrt(h), one layer
    __device__ __forceinline__ T &ih() const { return s[NV + 2]; } // 1/h, one layer
};

// One 8-byte LDS read kept as a single instruction.  On gfx950 the paired
// form the compiler otherwise makes of neighbouring fields (ds_read2_b64, two
// 8-byte values per lane) takes about 8 cycles per wavefront for consecutive
// records where a single read takes 2, and 22-30 against 7 for gathered ones:
// two single reads are about twice as fast.  A volatile read is not paired;
// it is made through an LDS pointer, since a volatile access through a
// generic one would stay a flat load.
template <typename T> __device__ __forceinline__ T lds(const T *p)
{
    return *(const volatile __attribute__((address_space(3))) T *)p;
}

// sqrt(h) and 1/h of a one-layer cell (the two-layer path keeps its LDS for
// occupancy and forms them per edge)
template <typename T, int NL, int NV> __device__ __forceinline__ void tri_cellpre(const TriCell<T, NL, NV> &c)
{
    if constexpr (NL == 1) {
        const T rq = FM<T>::rsq(c.s[0]);
        c.sq() = c.s[0] * rq;
        c.ih() = rq * rq;
    }
}

// Fluctuations |G| T^-1 (...) of both sides of a local edge between the
// cell records A and B (B == nullptr: a wall), in the x-y frame.  FX: the
// flux variant (FLUX_IR, FLUX_ROE, FLUX_IR_HH; two layers: FLUX_ROE or not).
template <typename T, int NL, bool TR, int NV, int FX = FLUX_IR>
__device__ __forceinline__ void tri_edge_flux(const TriCell<T, NL, NV> &CA, const TriCell<T, NL, NV> &CB, bool wall,
                                              T nx, T ny, T len, T g, T rr, T (&Fa)[NV], T (&Fb)[NV],
                                              unsigned &bad)
{
    const T *A = CA.s, *B = CB.s;
    if constexpr (NL == 1) {
        const T ha = lds(A), qxa = lds(A + 1), qya = lds(A + 2);
        const T ca = TR ? lds(A + 3) : T(0);
        const T qna = qxa * nx + qya * ny, qta = -qxa * ny + qya * nx;
        Flux1<T, TR> f;
        if (!wall) {
            const T hb = lds(B), qxb = lds(B + 1), qyb = lds(B + 2);
            const T cb = TR ? lds(B + 3) : T(0);
            const T qnb = qxb * nx + qyb * ny, qtb = -qxb * ny + qyb * nx;
            f = roe1_pre<T, TR, FX>(ha, lds(&CA.sq()), lds(&CA.ih()), qna, qta, ca, lds(&CA.z()), hb, lds(&CB.sq()),
                                lds(&CB.ih()), qnb, qtb, cb, lds(&CB.z()), g);
        } else {
            f = roe1_wall<T, TR>(ha, qna, qta, ca, g);
        }
        Fa[0] = len * f.am;
        Fa[1] = len * (f.an * nx - f.at * ny);
        Fa[2] = len * (f.an * ny + f.at * nx);
        Fb[0] = len * f.bm;
        Fb[1] = len * (f.bn * nx - f.bt * ny);
        Fb[2] = len * (f.bn * ny + f.bt * nx);
        if constexpr (TR) {
            Fa[3] = len * f.ac;
            Fb[3] = len * f.bc;
        }
    } else {
        T L[6], Rs[6];
#pragma unroll
        for (int l2 = 0; l2 < 2; ++l2) {
            const T qx = lds(A + 3 * l2 + 1), qy = lds(A + 3 * l2 + 2);
            L[3 * l2] = lds(A + 3 * l2);
            L[3 * l2 + 1] = qx * nx + qy * ny;
            L[3 * l2 + 2] = -qx * ny + qy * nx;
        }
        Flux2<T> f;
        if (!wall) {
#pragma unroll
            for (int l2 = 0; l2 < 2; ++l2) {
                const T qx = lds(B + 3 * l2 + 1), qy = lds(B + 3 * l2 + 2);
                Rs[3 * l2] = lds(B + 3 * l2);
                Rs[3 * l2 + 1] = qx * nx + qy * ny;
                Rs[3 * l2 + 2] = -qx * ny + qy * nx;
            }
            f = roe2_interior<T, flux_classical(FX)>(L, lds(&CA.z()), Rs, lds(&CB.z()), g, rr);
        } else {
            f = roe2_wall<T>(L, lds(&CA.z()), g, rr);
        }
        if (f.nonhyp) bad |= FLAG_NONHYPERBOLIC;
#pragma unroll
        for (int l2 = 0; l2 < 2; ++l2) {
            Fa[3 * l2] = len * f.a[3 * l2];
            Fa[3 * l2 + 1] = len * (f.a[3 * l2 + 1] * nx - f.a[3 * l2 + 2] * ny);
            Fa[3 * l2 + 2] = len * (f.a[3 * l2 + 1] * ny + f.a[3 * l2 + 2] * nx);
            Fb[3 * l2] = len * f.b[3 * l2];
            Fb[3 * l2 + 1] = len * (f.b[3 * l2 + 1] * nx - f.b[3 * l2 + 2] * ny);
            Fb[3 * l2 + 2] = len * (f.b[3 * l2 + 1] * ny + f.b[3 * l2 + 2] * nx);
        }
    }
}

// Eq. (5) speed |G| ||D||_inf of a local edge between cells CA and CB.
template <typename T, int NL, int NV>
__device__ __forceinline__ T tri_edge_speed(const TriCell<T, NL, NV> &CA, const TriCell<T, NL, NV> &CB, bool wall,
                                            T nx, T ny, T len, T g, T rr, unsigned &bad)
{
    const T *A = CA.s, *B = CB.s;
    T sp;
    if constexpr (NL == 1) {
        const T ha = lds(A), qna = lds(A + 1) * nx + lds(A + 2) * ny;
        if (!wall) {
            const T hb = lds(B), qnb = lds(B + 1) * nx + lds(B + 2) * ny;
            const T sa = lds(&CA.sq()), sb = lds(&CB.sq());
            // u_Roe = (sa ua + sb ub) / (sa + sb), s u = qn sqrt(h) / h
            const T ubar = (qna * sa * lds(&CA.ih()) + qnb * sb * lds(&CB.ih())) * FM<T>::rcp(sa + sb);
            sp = fabs(ubar) + FM<T>::sqrt(g * T(0.5) * (ha + hb));
        } else {
            sp = FM<T>::sqrt(g * ha);
        }
    } else {
        T L[6], Rs[6];
#pragma unroll
        for (int l2 = 0; l2 < 2; ++l2) {
            L[3 * l2] = lds(A + 3 * l2);
            L[3 * l2 + 1] = lds(A + 3 * l2 + 1) * nx + lds(A + 3 * l2 + 2) * ny;
            L[3 * l2 + 2] = T(0);
        }
        T pa[4], pb[4];
        roe2_cellpre(L, pa);
        if (!wall) {
#pragma unroll
            for (int l2 = 0; l2 < 2; ++l2) {
                Rs[3 * l2] = lds(B + 3 * l2);
                Rs[3 * l2 + 1] = lds(B + 3 * l2 + 1) * nx + lds(B + 3 * l2 + 2) * ny;
                Rs[3 * l2 + 2] = T(0);
            }
            roe2_cellpre(Rs, pb);
        } else { // mirror state
            Rs[0] = L[0];
            Rs[1] = -L[1];
            Rs[3] = L[3];
            Rs[4] = -L[4];
            Rs[2] = Rs[5] = T(0);
#pragma unroll
            for (int q = 0; q < 4; ++q) pb[q] = pa[q];
        }
        bool nh2 = false;
        sp = roe2_speed<T>(L, pa, Rs, pb, g, rr, nh2);
        if (nh2) bad |= FLAG_NONHYPERBOLIC;
    }
    return len * sp;
}

// Element i of an array through a 32-bit byte offset (scalar base plus
// vector offset addressing; every array of this path is below 4 GiB: cells
// and local edges < 2^29).
template <typename T> __device__ __forceinline__ const T &ld32(const T *base, uint32_t i)
{
    return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + (uint32_t)(i * (uint32_t)sizeof(T)));
}
template <typename T> __device__ __forceinline__ T &st32(T *base, uint32_t i)
{
    return *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + (uint32_t)(i * (uint32_t)sizeof(T)));
}

// Per-step bookkeeping by workgroup 0: clear the partial-minimum bank and
// the block counters the launch after next will use, record dt^n and
// advance the time.
template <typename T> __device__ __forceinline__ void tri_book(const TriArgs<T> &A, int bank, int tid, double dtd)
{
    if (tid < 64) {
        A.part[((bank + 2) % 3) * TRI_NPART + tid] = __builtin_inf();
        if (tid < TRI_XCD) A.ctr[(((bank + 2) % 3) * TRI_XCD + tid) * TRI_CTR_STRIDE] = 0u;
        if (tid == 0) {
            A.book.hist[A.step] = dtd;
            A.book.last[0] = dtd;
            A.book.t[0] += dtd;
        }
    }
}

// An edge's packed cell pair (a | b << 16) in a real-valued LDS slot, exact.
__device__ __forceinline__ float tri_pack(uint32_t v, float) { return __uint_as_float(v); }
__device__ __forceinline__ double tri_pack(uint32_t v, double) { return (double)v; }
__device__ __forceinline__ uint32_t tri_unpack(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t tri_unpack(double x) { return (uint32_t)x; }

// RD: rounds of NT threads covering the largest local cell / edge / slot
// counts of any block.  Every global load a thread will need in the launch
// (halo ids, its edges' geometry, its cells' slot lists and 1/|V|) is issued
// at the start, so the phases after the first barrier only touch LDS.
//
// RC: the recomputation variant.  Instead of evaluating each local edge
// once into LDS records that its two cells gather, every cell evaluates all
// three of its edges itself (interior edges twice over), for the fluxes and
// for the Eq. (5) speeds; the LDS edge records then hold the edges' cell
// pair and geometry.  Same inputs per edge, same accumulation order.
// Two layers (shared edges): at least four waves per SIMD, so that two
// 512-thread workgroups fit a CU (LDS allows two 224-cell blocks); the
// classical flux would otherwise take 142 VGPRs and leave room for one.
template <typename T, int NL, bool TR, bool DT0, int RD, int NT, int FX = FLUX_IR, bool RC = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NL == 2 && !RC ? 4 : 1))) void
k_tri_fused(TriArgs<T> A)
{
    constexpr int NV = NL == 2 ? 6 : (TR ? 4 : 3);
    using Rec = TriRec<NL, NV>;
    using Cell = TriCell<T, NL, NV>;
    constexpr int ER = Rec::ER;
    extern __shared__ double smem_d[];
    T *sm = reinterpret_cast<T *>(smem_d); // cell records
    const int LCM = A.lc_max, EM = A.e_max;
    T *fl = sm + (Rec::SA + Rec::AX) * LCM; // side s, var v of edge e at fl[s ER EM + ER e + v]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = blockIdx.x;
    const int blk = (w % TRI_XCD) * A.per_xcd + w / TRI_XCD;
    const int bank = (int)((A.step + A.bank0) % 3);
    // the partial minima of dt^n: loaded now, reduced when the update needs
    // them, so their latency overlaps the block's own loads
    const double dpart = DT0 ? 0.0 : A.part[bank * TRI_NPART + lane];
    if (blk >= A.nblocks) { // uniform over the workgroup
        if (!DT0 && w == 0) tri_book(A, bank, tid, wave_min(dpart));
        return;
    }

    const int64_t base = (int64_t)blk * A.B;
    const int B0 = (int)min((int64_t)A.B, A.N - base);
    const int h0 = A.halo_off[blk], nh = A.halo_off[blk + 1] - h0;
    const int n1 = A.n1[blk];
    const int LC = B0 + nh;
    const int e0 = A.edge_off[blk], ne = A.edge_off[blk + 1] - e0, es0 = A.e_s0[blk];
    const int s0 = A.slot_off[blk];
    const int nc = B0 + n1; // cells updated (block + ring 1)
    const T g = A.g, rr = A.r;
    unsigned bad = 0;

    // ---- all global reads of the launch, issued up front.  The loads are
    // unconditional (indices clamped into the block's ranges, which are never
    // empty, and the halo list ends with a padding entry) and out-of-range
    // lanes are masked afterwards, so no load waits on a branch.
    const uint32_t ubase = (uint32_t)base;
    const int nh1 = max(nh - 1, 0);
    const int ne1 = (DT0 ? es0 : ne) - 1, nc1 = nc - 1;
    int32_t hid[RD];
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const int l = tid + m * NT;
        hid[m] = ld32(A.halo_ids, (uint32_t)(h0 + min(max(l - B0, 0), nh1)));
    }
    uint32_t eab[RD];
    T enx[RD], eny[RD], elen[RD];
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const uint32_t k = (uint32_t)(e0 + min(tid + m * NT, ne1));
        eab[m] = ld32(A.e_ab, k);
        enx[m] = ld32(A.e_gx, k); // |G| eta until the loads land
        eny[m] = ld32(A.e_gy, k);
    }
    uint64_t csl4[RD];
    T cia[RD];
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const uint32_t r = (uint32_t)(s0 + min(tid + m * NT, nc1));
        csl4[m] = ld32(reinterpret_cast<const uint64_t *>(A.slots), r);
        cia[m] = ld32(A.iarea, r);
    }
    // (an empty asm use pins the halo-id loads here, ahead of the selection
    // below, which would otherwise pull them into a branch and wait on each)
#pragma unroll
    for (int m = 0; m < RD; ++m) asm volatile("" ::"v"(hid[m]));
    uint32_t gidx[RD]; // a valid cell for every lane; only l < LC are local cells (record offsets NV * cell)
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const int l = tid + m * NT;
        gidx[m] = l < B0 ? ubase + (uint32_t)l : (uint32_t)hid[m];
    }

    // ---- 1. W^n and z of the block and its two rings into LDS (all rounds
    // loaded before the first LDS write)
    T st[RD][NV + 1];
#pragma unroll
    for (int m = 0; m < RD; ++m) {
#pragma unroll
        for (int v = 0; v < NV; ++v) st[m][v] = ld32(A.in, gidx[m] * NV + v);
        st[m][NV] = ld32(A.z, gidx[m]);
    }
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const int l = tid + m * NT;
        if (l < LC) {
            const Cell c(sm, LCM, l);
#pragma unroll
            for (int v = 0; v < NV; ++v) c.s[v] = st[m][v];
            c.z() = st[m][NV];
            tri_cellpre<T, NL, NV>(c);
        }
    }
    // unit normal and length of each of this thread's edges from |G| eta
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const T q = enx[m] * enx[m] + eny[m] * eny[m];
        const T rq = FM<T>::rsq(q);
        elen[m] = q * rq;
        enx[m] *= rq;
        eny[m] *= rq;
    }
    if constexpr (RC && !DT0) { // edge records: cell pair, normal (side 0), length (side 1)
#pragma unroll
        for (int m = 0; m < RD; ++m) {
            const int k = tid + m * NT;
            if (k < ne) {
                T *fa = fl + ER * k;
                fa[0] = tri_pack(eab[m], T(0));
                fa[1] = enx[m];
                fa[2] = eny[m];
                fl[ER * (EM + k)] = elen[m];
            }
        }
    }
    // the edge of a slot, from the records above (RC)
    auto slot_edge = [&](unsigned sl, int &la, int &lb, bool &wall, T &nx, T &ny, T &len, bool &side_b) {
        const unsigned q = sl / (unsigned)ER;
        side_b = q >= (unsigned)EM;
        const unsigned k = side_b ? q - (unsigned)EM : q;
        const T *fa = fl + ER * k;
        const uint32_t ab = tri_unpack(fa[0]);
        nx = fa[1];
        ny = fa[2];
        len = fl[ER * (EM + k)];
        la = (int)(ab & 0xFFFFu);
        lb = (int)(ab >> 16);
        wall = lb == 0xFFFF;
        if (wall) lb = 0;
    };
    __syncthreads();

    double dtd = 0.0;
    if constexpr (!DT0 && RC) {
        // ---- 2-3 (RC). W^{n+1} of the block and ring 1, every cell
        // evaluating its three edges itself; the new states wait in
        // registers until every thread has read W^n
        dtd = wave_min(dpart);
        T nw[RD][NV];
#pragma unroll
        for (int m = 0; m < RD; ++m) {
            const int l = tid + m * NT;
            if (l < nc) {
                T acc[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] = T(0);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    int la, lb;
                    bool wall, sb;
                    T nx, ny, len;
                    slot_edge((unsigned)(csl4[m] >> (16 * j)) & 0xFFFFu, la, lb, wall, nx, ny, len, sb);
                    T Fa[NV], Fb[NV];
                    tri_edge_flux<T, NL, TR, NV, FX>(Cell(sm, LCM, la), Cell(sm, LCM, lb), wall, nx, ny, len, g, rr,
                                                     Fa, Fb, bad);
#pragma unroll
                    for (int v = 0; v < NV; ++v) acc[v] += sb ? Fb[v] : Fa[v];
                }
                const T fct = (T)dtd * cia[m];
                const Cell c(sm, LCM, l);
#pragma unroll
                for (int v = 0; v < NV; ++v) nw[m][v] = lds(c.s + v) - fct * acc[v];
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < RD; ++m) {
            const int l = tid + m * NT;
            if (l < nc) {
                const Cell c(sm, LCM, l);
#pragma unroll
                for (int v = 0; v < NV; ++v) c.s[v] = nw[m][v];
                tri_cellpre<T, NL, NV>(c);
            }
        }
        __syncthreads();
    } else if (!DT0) {
        // ---- 2. every edge touching the block or ring 1, once
#pragma unroll
        for (int m = 0; m < RD; ++m) {
            const int k = tid + m * NT;
            if (k < ne) {
                const unsigned lb = eab[m] >> 16;
                const bool wall = lb == 0xFFFFu;
                T Fa[NV], Fb[NV];
                tri_edge_flux<T, NL, TR, NV, FX>(Cell(sm, LCM, (int)(eab[m] & 0xFFFFu)), Cell(sm, LCM, wall ? 0 : (int)lb),
                                             wall, enx[m], eny[m], elen[m], g, rr, Fa, Fb, bad);
                T *fa = fl + ER * k, *fb = fl + ER * (EM + k);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    fa[v] = Fa[v];
                    fb[v] = Fb[v];
                }
            }
        }
        __syncthreads();

        dtd = wave_min(dpart);
        // ---- 3. W^{n+1} of the block and ring 1, gathered in a fixed order
        // (a slot is the offset of a side's record: (side EM + edge) ER)
#pragma unroll
        for (int m = 0; m < RD; ++m) {
            const int l = tid + m * NT;
            if (l < nc) {
                T acc[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] = T(0);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const T *f = fl + ((unsigned)(csl4[m] >> (16 * j)) & 0xFFFFu);
#pragma unroll
                    for (int v = 0; v < NV; ++v) acc[v] += lds(f + v);
                }
                const T fct = (T)dtd * cia[m];
                const Cell c(sm, LCM, l);
#pragma unroll
                for (int v = 0; v < NV; ++v) c.s[v] -= fct * acc[v];
                tri_cellpre<T, NL, NV>(c);
            }
        }
        __syncthreads();
    }

    // ---- 4. Eq. (5) speeds on the edges touching the block (of W^{n+1}, or
    // of W^0 for the prologue), parked at both sides' first slot so that the
    // cells' slots address them directly
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const int k = tid + m * NT;
        if (!(RC && !DT0) && k < es0) {
            const unsigned lb = eab[m] >> 16;
            const bool wall = lb == 0xFFFFu;
            const T sp = tri_edge_speed<T, NL, NV>(Cell(sm, LCM, (int)(eab[m] & 0xFFFFu)),
                                                   Cell(sm, LCM, wall ? 0 : (int)lb), wall, enx[m], eny[m], elen[m],
                                                   g, rr, bad);
            fl[ER * k] = sp;
            fl[ER * (EM + k)] = sp;
        }
    }
    if constexpr (!(RC && !DT0)) __syncthreads();

    // ---- 5. dt candidates of the block cells, W^{n+1} out.  dt_i =
    // 2 gamma / (S_i / |V_i|) and a correctly rounded quotient is monotone in
    // its divisor, so the smallest dt_i is 2 gamma over the largest S_i / |V_i|.
    T rate = T(0);
#pragma unroll
    for (int m = 0; m < RD; ++m) {
        const int l = tid + m * NT;
        if (l < B0) {
            T S;
            if constexpr (RC && !DT0) { // the cell's three edge speeds, evaluated here
                T sp[3];
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    int la, lb;
                    bool wall, sb;
                    T nx, ny, len;
                    slot_edge((unsigned)(csl4[m] >> (16 * j)) & 0xFFFFu, la, lb, wall, nx, ny, len, sb);
                    sp[j] = tri_edge_speed<T, NL, NV>(Cell(sm, LCM, la), Cell(sm, LCM, lb), wall, nx, ny, len, g, rr,
                                                      bad);
                }
                S = sp[0] + sp[1] + sp[2];
            } else {
                S = fl[(unsigned)csl4[m] & 0xFFFFu] + fl[(unsigned)(csl4[m] >> 16) & 0xFFFFu] +
                    fl[(unsigned)(csl4[m] >> 32) & 0xFFFFu];
            }
            rate = fmax(rate, cia[m] * S);
            if (!DT0) {
                bool badv = false;
                const T *c = sm + l * Rec::SA;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const T x = c[v];
                    st32(A.out, (ubase + (uint32_t)l) * NV + v) = x;
                    badv |= !isfinite(x);
                }
                if (!(c[0] > T(0)) || (NL == 2 && !(c[3] > T(0)))) bad |= FLAG_DEPTH;
                if (badv) bad |= FLAG_NONFINITE;
            }
        }
    }
    const double cand = rate > T(0) ? (double)(T(2) * A.cfl / rate) : __builtin_inf();
    const int slot_bank = DT0 ? 0 : (bank + 1) % 3;
    block_min_to_slot(cand, A.part + slot_bank * TRI_NPART + (w % TRI_NPART));
    if (bad) atomicOr(A.book.flags, bad);
    if (!DT0 && w == 0) tri_book(A, bank, tid, dtd);
}

// ---------------------------------------------------------------------------
// Software-pipelined variant: a persistent workgroup walks a band of blocks
// and, while it evaluates block i, already has block i+1's global reads in
// flight (its scalars, halo ids, edge data and slot rows during the flux
// phase; its cell states during the update and speed phases).  One round of
// threads covers a block (local cells, edges and updated cells <= NT).
// ---------------------------------------------------------------------------

// Scalars of one block.
struct TriBlk {
    int base, B0, h0, nh, n1, e0, ne, es0, s0;
};

template <typename T> __device__ __forceinline__ TriBlk tri_blk(const TriArgs<T> &A, int blk)
{
    TriBlk b;
    b.base = blk * A.B; // cells < 2^29
    b.B0 = min(A.B, (int)A.N - b.base);
    b.h0 = A.halo_off[blk];
    b.nh = A.halo_off[blk + 1] - b.h0;
    b.n1 = A.n1[blk];
    b.e0 = A.edge_off[blk];
    b.ne = A.edge_off[blk + 1] - b.e0;
    b.es0 = A.e_s0[blk];
    b.s0 = A.slot_off[blk];
    return b;
}

// One thread's reads of a block's mesh data: its halo id, its edge (local
// id pair, |G| eta), its cell's slot row and 1/|V| (indices clamped into the
// block's ranges; out-of-range threads are masked where the values are used).
template <typename T> struct TriPre {
    int32_t hid;
    uint32_t eab;
    T gx, gy;
    uint32_t csl; // three 10-bit fluctuation-record indices
    T cia;
};

template <typename T> __device__ __forceinline__ TriPre<T> tri_pre(const TriArgs<T> &A, const TriBlk &b, int tid)
{
    TriPre<T> p;
    p.hid = ld32(A.halo_ids, (uint32_t)(b.h0 + min(max(tid - b.B0, 0), max(b.nh - 1, 0))));
    const uint32_t k = (uint32_t)(b.e0 + min(tid, b.ne - 1));
    p.eab = ld32(A.e_ab, k);
    p.gx = ld32(A.e_gx, k);
    p.gy = ld32(A.e_gy, k);
    const uint32_t r = (uint32_t)(b.s0 + min(tid, b.B0 + b.n1 - 1));
    p.csl = ld32(A.slots32, r);
    p.cia = ld32(A.iarea, r);
    return p;
}

// The thread's local cell of a block: W^n and z (a valid cell for every
// thread; only tid < B0 + nh are local cells).
template <typename T, int NV>
__device__ __forceinline__ void tri_state(const TriArgs<T> &A, const TriBlk &b, const TriPre<T> &p, int tid,
                                          T (&st)[NV + 1])
{
    const uint32_t gi = tid < b.B0 ? (uint32_t)(b.base + tid) : (uint32_t)p.hid;
#pragma unroll
    for (int v = 0; v < NV; ++v) st[v] = ld32(A.in, gi * NV + v);
    st[NV] = ld32(A.z, gi);
}

template <typename T, int NL, bool TR, int NT, int FX = FLUX_IR>
__global__ __launch_bounds__(NT) void k_tri_pipe(TriArgs<T> A)
{
    constexpr int NV = NL == 2 ? 6 : (TR ? 4 : 3);
    using Rec = TriRec<NL, NV>;
    using Cell = TriCell<T, NL, NV>;
    constexpr int ER = Rec::ER;
    extern __shared__ double smem_d[];
    T *sm = reinterpret_cast<T *>(smem_d);
    const int LCM = A.lc_max, EM = A.e_max;
    T *fl = sm + (Rec::SA + Rec::AX) * LCM;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = blockIdx.x;
    const int bank = (int)((A.step + A.bank0) % 3);
    // XCD-aware: the G workgroups of XCD w % 8 share its band of consecutive
    // (Morton-neighbouring) blocks.  Each takes the band positions w / 8 and
    // w / 8 + G, then further positions from 2 G on, one at a time, from the
    // band's counter: the resident workgroups of a CU do not progress at the
    // same rate (on the 2M mesh a CU's first workgroup spent 3.4 us per block,
    // its third 5.9), and a fixed deal of the band left the slowest finishing
    // last.  Every other step walks the band backwards, so that it begins with
    // the blocks its predecessor wrote last.
    const int xcd = w % TRI_XCD, G = (int)gridDim.x / TRI_XCD;
    const int bstart = xcd * A.per_xcd;
    const int nband = min(A.per_xcd, A.nblocks - bstart);
    unsigned *const ctr = A.ctr + (bank * TRI_XCD + xcd) * TRI_CTR_STRIDE;
    __shared__ int s_next; // the next position, published in the previous block's phase 5
    int pos = w / TRI_XCD, npos = pos + G;
    bool first = true;
    const double dpart = A.part[bank * TRI_NPART + lane];
    const T g = A.g, rr = A.r;
    unsigned bad = 0;
    T rate = T(0);

    TriBlk cb{};
    TriPre<T> cp{};
    T cst[NV + 1];
#pragma unroll
    for (int v = 0; v <= NV; ++v) cst[v] = T(1);
    if (pos < nband) {
        cb = tri_blk(A, A.rev ? bstart + nband - 1 - pos : bstart + pos);
        cp = tri_pre(A, cb, tid);
        asm volatile("" ::"v"(cp.hid));
        tri_state<T, NV>(A, cb, cp, tid, cst);
    }
    const double dtd = wave_min(dpart);

    while (pos < nband) { // uniform over the workgroup
        const int LC = cb.B0 + cb.nh, nc = cb.B0 + cb.n1;

        // ---- 1. W^n and z into LDS; this thread's edge geometry
        if (tid < LC) {
            const Cell c(sm, LCM, tid);
#pragma unroll
            for (int v = 0; v < NV; ++v) c.s[v] = cst[v];
            c.z() = cst[NV];
            tri_cellpre<T, NL, NV>(c);
        }
        const T q = cp.gx * cp.gx + cp.gy * cp.gy;
        const T rq = FM<T>::rsq(q);
        const T elen = q * rq, enx = cp.gx * rq, eny = cp.gy * rq;
        const unsigned la = cp.eab & 0xFFFFu, lb = cp.eab >> 16;
        const bool wall = lb == 0xFFFFu;
        __syncthreads();
        if (!first) npos = s_next; // rewritten only in this block's phase 5
        first = false;
        const bool more = npos < nband;

        // next block's scalars and mesh data.  Issued on every pass (the
        // current block again once the band is done): with a branch around
        // them, the compiler's wait counters merged the path without loads
        // into the flux phase and made it wait for these loads to return
        const int lpos = more ? npos : pos;
        const TriBlk nb = tri_blk(A, A.rev ? bstart + nband - 1 - lpos : bstart + lpos);
        const TriPre<T> np = tri_pre(A, nb, tid);

        // ---- 2. every edge touching the block or ring 1, once
        if (tid < cb.ne) {
            T Fa[NV], Fb[NV];
            tri_edge_flux<T, NL, TR, NV, FX>(Cell(sm, LCM, (int)la), Cell(sm, LCM, wall ? 0 : (int)lb), wall, enx, eny,
                                         elen, g, rr, Fa, Fb, bad);
            T *fa = fl + ER * tid, *fb = fl + ER * (EM + tid);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                fa[v] = Fa[v];
                fb[v] = Fb[v];
            }
        }
        __syncthreads();

        // the position after next, from the band's counter, by the last wave:
        // the compiler waits for the returned value right away, and with 224-
        // cell blocks on 512 threads that wave has no cell or edge in phases
        // 3 to 5 (its state loads below are placeholders)
        unsigned taken = 0;
        if (more && tid == NT - 64) taken = atomicAdd(ctr, 1u);

        // next block's cell states (its halo ids have arrived)
        T nst[NV + 1];
        tri_state<T, NV>(A, nb, np, tid, nst);

        // ---- 3. W^{n+1} of the block and ring 1, gathered in a fixed order;
        // the block's own cells go out to HBM from registers right away, so
        // that phase 5 reads no cell record and the next block may refill
        // them without another barrier
        if (tid < nc) {
            T acc[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[v] = T(0);
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const T *f = fl + ER * ((cp.csl >> (10 * j)) & 0x3FFu);
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] += lds(f + v);
            }
            const T fct = (T)dtd * cp.cia;
            const Cell c(sm, LCM, tid);
            T nw[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                nw[v] = lds(c.s + v) - fct * acc[v];
                c.s[v] = nw[v];
            }
            tri_cellpre<T, NL, NV>(c);
            if (tid < cb.B0) {
                bool badv = false;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    st32(A.out, (uint32_t)(cb.base + tid) * NV + v) = nw[v];
                    badv |= !isfinite(nw[v]);
                }
                if (!(nw[0] > T(0)) || (NL == 2 && !(nw[3] > T(0)))) bad |= FLAG_DEPTH;
                if (badv) bad |= FLAG_NONFINITE;
            }
        }
        __syncthreads();

        // ---- 4. Eq. (5) speeds of W^{n+1} on the edges touching the block
        if (tid < cb.es0) {
            const T sp = tri_edge_speed<T, NL, NV>(Cell(sm, LCM, (int)la), Cell(sm, LCM, wall ? 0 : (int)lb), wall,
                                                   enx, eny, elen, g, rr, bad);
            fl[ER * tid] = sp;
            fl[ER * (EM + tid)] = sp;
        }
        __syncthreads();

        // ---- 5. the block cells' S_i / |V_i|.  No barrier follows: this
        // phase reads only the speed slots, which the next block writes after
        // its first barrier, and the next block's phase 1 fills only the cell
        // records
        if (tid < cb.B0) {
            const T S = fl[ER * (cp.csl & 0x3FFu)] + fl[ER * ((cp.csl >> 10) & 0x3FFu)] +
                        fl[ER * ((cp.csl >> 20) & 0x3FFu)];
            rate = fmax(rate, cp.cia * S);
        }
        if (tid == NT - 64) s_next = more ? 2 * G + (int)taken : nband; // read after the next first barrier

        cb = nb;
        cp = np;
#pragma unroll
        for (int v = 0; v <= NV; ++v) cst[v] = nst[v];
        pos = npos;
    }

    // dt candidate of everything this workgroup updated: 2 gamma over the
    // largest S_i / |V_i| (a correctly rounded quotient is monotone)
    const double cand = rate > T(0) ? (double)(T(2) * A.cfl / rate) : __builtin_inf();
    block_min_to_slot(cand, A.part + ((bank + 1) % 3) * TRI_NPART + (w % TRI_NPART));
    if (bad) atomicOr(A.book.flags, bad);
    if (w == 0) tri_book(A, bank, tid, dtd);
}

// Batch start: elapsed time, error flags and every block counter to zero;
// the partial minima too when the batch starts from a fresh state (as
// k_cart_init).
__global__ void k_tri_init(double *part, StepBook book, int reset_part)
{
    const int t = threadIdx.x;
    if (reset_part)
        for (int k = t; k < 3 * TRI_NPART; k += blockDim.x) part[k] = __builtin_inf();
    if (t < 3 * TRI_XCD) reinterpret_cast<unsigned *>(part + 3 * TRI_NPART)[t * TRI_CTR_STRIDE] = 0u;
    if (t == 0) {
        book.t[0] = 0.0;
        book.flags[0] = 0u;
    }
}

// caller order <-> internal (Morton) order
template <typename T>
__global__ void k_permute(const T *__restrict__ src, T *__restrict__ dst, const int32_t *__restrict__ perm,
                          int64_t n, int to_internal)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (to_internal) dst[i] = src[perm[i]];
    else dst[perm[i]] = src[i];
}

hipError_t launch_permute(swe_ctx *c, const void *src, void *dst, int to_internal)
{
    const unsigned nb = (unsigned)((c->N + 255) / 256);
    if (c->prec == SWE_F32)
        hipLaunchKernelGGL(k_permute<float>, dim3(nb), dim3(256), 0, c->stream, (const float *)src, (float *)dst,
                           c->perm, c->N, to_internal);
    else
        hipLaunchKernelGGL(k_permute<double>, dim3(nb), dim3(256), 0, c->stream, (const double *)src,
                           (double *)dst, c->perm, c->N, to_internal);
    return hipGetLastError();
}

// The caller's separate arrays, in the caller's cell order <-> the records
// of the fused triangle path, in internal (Morton) order: record i holds the
// nv variables of caller cell perm[i].
template <typename T>
__global__ void k_tri_pack(const int32_t *__restrict__ perm, StatePtrs<T> soa, T *__restrict__ rec, int64_t n, int nv,
                           int pack)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t k = perm[i];
    for (int v = 0; v < nv; ++v) {
        if (pack) rec[i * nv + v] = soa.v[v][k];
        else soa.v[v][k] = rec[i * nv + v];
    }
}

template <typename T> static hipError_t tri_pack_t(swe_ctx *c, const void *const *soa, void *rec, int pack)
{
    StatePtrs<T> p;
    for (int v = 0; v < 6; ++v) p.v[v] = v < c->nv ? (T *)soa[v] : nullptr;
    const unsigned nb = (unsigned)((c->N + 255) / 256);
    hipLaunchKernelGGL(k_tri_pack<T>, dim3(nb), dim3(256), 0, c->stream, c->perm, p, (T *)rec, c->N, c->nv, pack);
    return hipGetLastError();
}

hipError_t launch_tri_pack(swe_ctx *c, const void *const *soa, void *rec, int pack)
{
    return c->prec == SWE_F32 ? tri_pack_t<float>(c, soa, rec, pack) : tri_pack_t<double>(c, soa, rec, pack);
}

template <typename T> static TriArgs<T> tri_args(swe_ctx *c, int64_t step, double cfl)
{
    TriArgs<T> A;
    const int in = c->cur ^ (int)(step & 1), out = in ^ 1;
    A.in = (const T *)c->state[in];
    A.out = (T *)c->state[out];
    A.z = (const T *)c->zbed;
    A.N = c->N;
    A.B = c->tb.B;
    A.nblocks = c->tb.nblocks;
    A.per_xcd = (A.nblocks + TRI_XCD - 1) / TRI_XCD;
    A.lc_max = c->tb.lc_max;
    A.e_max = c->tb.e_max;
    A.halo_off = c->tb.halo_off;
    A.halo_ids = c->tb.halo_ids;
    A.n1 = c->tb.n1;
    A.edge_off = c->tb.edge_off;
    A.e_s0 = c->tb.e_s0;
    A.slot_off = c->tb.slot_off;
    A.e_ab = c->tb.e_ab;
    A.e_gx = (const T *)c->tb.e_gx;
    A.e_gy = (const T *)c->tb.e_gy;
    A.slots = c->tb.slots;
    A.slots32 = c->tb.slots32;
    A.iarea = (const T *)c->tb.iarea;
    A.g = (T)c->g;
    A.r = (T)c->r;
    A.cfl = (T)cfl;
    A.part = c->cart_part;
    A.ctr = reinterpret_cast<unsigned *>(c->cart_part + 3 * TRI_NPART);
    A.rev = in; // the step that reads the second state buffer walks backwards
    A.book = c->book;
    A.step = step;
    A.bank0 = c->bank0;
    return A;
}

// FX: the flux variant.  The initial-state dt prologue computes speeds
// only, which both fluxes share, so it is the IR-Roe instance.
template <typename T, int NL, bool TR, int RD, int NT, int FX, bool RC = false>
static hipError_t tri_batch_rd(swe_ctx *c, int32_t nsteps, double cfl)
{
    constexpr int NV = NL == 2 ? 6 : (TR ? 4 : 3);
    const size_t lds = tri_lds_bytes(NV, sizeof(T), c->tb.lc_max, c->tb.e_max);
    const int per_xcd = (c->tb.nblocks + TRI_XCD - 1) / TRI_XCD;
    const dim3 grid((unsigned)(per_xcd * TRI_XCD)), block(NT);
    if (lds > 65536) { // above the default dynamic LDS limit: opt in per kernel
        hipError_t e = hipFuncSetAttribute((const void *)k_tri_fused<T, NL, TR, true, RD, NT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute((const void *)k_tri_fused<T, NL, TR, false, RD, NT, FX, RC>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    // dt of the current state: left by the previous batch (same state, same
    // cfl), else computed here into bank 0 (the prologue writes bank 0)
    const bool fresh = !c->dt_ready || c->dt_cfl != cfl;
    if (fresh) c->bank0 = 0;
    hipLaunchKernelGGL(k_tri_init, dim3(1), dim3(64), 0, c->stream, c->cart_part, c->book, fresh ? 1 : 0);
    if (fresh)
        hipLaunchKernelGGL((k_tri_fused<T, NL, TR, true, RD, NT>), grid, block, lds, c->stream,
                           tri_args<T>(c, 0, cfl));
    if constexpr (RD == 1 && !RC) {
        if (c->tb.pipe_wgs != 0) {
            if (lds > 65536) {
                const hipError_t e = hipFuncSetAttribute((const void *)k_tri_pipe<T, NL, TR, NT, FX>,
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e != hipSuccess) return e;
            }
            int per_cu = 0;
            if (c->tb.pipe_wgs < 0) { // as many workgroups as can be resident at once
                int cus = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_tri_pipe<T, NL, TR, NT, FX>, NT, lds) !=
                        hipSuccess ||
                    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device) != hipSuccess)
                    return hipErrorUnknown;
                c->tb.pipe_wgs = std::max(1, per_cu) * std::max(1, cus);
            }
            const dim3 pgrid((unsigned)(TRI_XCD * std::max(1, std::min(c->tb.pipe_wgs / TRI_XCD, per_xcd))));
            if (per_cu > 0) // sized just now: the description names the grid
                c->desc += ", " + std::to_string(pgrid.x) + " persistent workgroups (" + std::to_string(per_cu) +
                           " resident per CU)";
            for (int64_t s = 0; s < nsteps; ++s)
                hipLaunchKernelGGL((k_tri_pipe<T, NL, TR, NT, FX>), pgrid, block, lds, c->stream, tri_args<T>(c, s, cfl));
            return hipGetLastError();
        }
    }
    for (int64_t s = 0; s < nsteps; ++s)
        hipLaunchKernelGGL((k_tri_fused<T, NL, TR, false, RD, NT, FX, RC>), grid, block, lds, c->stream,
                           tri_args<T>(c, s, cfl));
    return hipGetLastError();
}

template <typename T, int NL, bool TR, int FX = FLUX_IR>
static hipError_t tri_batch_t(swe_ctx *c, int32_t nsteps, double cfl)
{
    // 512 threads per workgroup (eight wavefronts: the block's latency is
    // hidden by its own waves as much as by the other blocks on the CU);
    // rounds of threads cover the largest local cell / edge / update counts
    // (checked at create)
    if (c->tb.nt == 512) {
        if (c->tb.rounds <= 1) return tri_batch_rd<T, NL, TR, 1, 512, FX>(c, nsteps, cfl);
        return tri_batch_rd<T, NL, TR, 2, 512, FX>(c, nsteps, cfl);
    }
    if (c->tb.rounds <= 1) return tri_batch_rd<T, NL, TR, 1, 256, FX>(c, nsteps, cfl);
    if (c->tb.rounds <= 2) return tri_batch_rd<T, NL, TR, 2, 256, FX>(c, nsteps, cfl);
    return tri_batch_rd<T, NL, TR, 3, 256, FX>(c, nsteps, cfl);
}

// The recomputation variant (IR-Roe, 512 threads per workgroup).
template <typename T, int NL, bool TR> static hipError_t tri_batch_rc(swe_ctx *c, int32_t nsteps, double cfl)
{
    if (c->tb.rounds <= 1) return tri_batch_rd<T, NL, TR, 1, 512, false, true>(c, nsteps, cfl);
    return tri_batch_rd<T, NL, TR, 2, 512, false, true>(c, nsteps, cfl);
}

hipError_t launch_tri_batch(swe_ctx *c, int32_t nsteps, double cfl)
{
    const bool f32 = c->prec == SWE_F32;
    if (c->path == SWE_PATH_RECOMPUTE) { // IR-Roe only
        if (c->nlayers == 2) return f32 ? tri_batch_rc<float, 2, false>(c, nsteps, cfl) : tri_batch_rc<double, 2, false>(c, nsteps, cfl);
        if (c->ntracers) return f32 ? tri_batch_rc<float, 1, true>(c, nsteps, cfl) : tri_batch_rc<double, 1, true>(c, nsteps, cfl);
        return f32 ? tri_batch_rc<float, 1, false>(c, nsteps, cfl) : tri_batch_rc<double, 1, false>(c, nsteps, cfl);
    }
    if (c->nlayers == 2) {
        if (c->classical)
            return f32 ? tri_batch_t<float, 2, false, FLUX_ROE>(c, nsteps, cfl) : tri_batch_t<double, 2, false, FLUX_ROE>(c, nsteps, cfl);
        return f32 ? tri_batch_t<float, 2, false>(c, nsteps, cfl) : tri_batch_t<double, 2, false>(c, nsteps, cfl);
    }
    if (c->classical && c->hh) {
        if (c->ntracers)
            return f32 ? tri_batch_t<float, 1, true, FLUX_ROE_HH>(c, nsteps, cfl) : tri_batch_t<double, 1, true, FLUX_ROE_HH>(c, nsteps, cfl);
        return f32 ? tri_batch_t<float, 1, false, FLUX_ROE_HH>(c, nsteps, cfl) : tri_batch_t<double, 1, false, FLUX_ROE_HH>(c, nsteps, cfl);
    }
    if (c->classical) {
        if (c->ntracers)
            return f32 ? tri_batch_t<float, 1, true, FLUX_ROE>(c, nsteps, cfl) : tri_batch_t<double, 1, true, FLUX_ROE>(c, nsteps, cfl);
        return f32 ? tri_batch_t<float, 1, false, FLUX_ROE>(c, nsteps, cfl) : tri_batch_t<double, 1, false, FLUX_ROE>(c, nsteps, cfl);
    }
    if (c->hh) {
        if (c->ntracers)
            return f32 ? tri_batch_t<float, 1, true, FLUX_IR_HH>(c, nsteps, cfl) : tri_batch_t<double, 1, true, FLUX_IR_HH>(c, nsteps, cfl);
        return f32 ? tri_batch_t<float, 1, false, FLUX_IR_HH>(c, nsteps, cfl) : tri_batch_t<double, 1, false, FLUX_IR_HH>(c, nsteps, cfl);
    }
    if (c->ntracers) return f32 ? tri_batch_t<float, 1, true>(c, nsteps, cfl) : tri_batch_t<double, 1, true>(c, nsteps, cfl);
    return f32 ? tri_batch_t<float, 1, false>(c, nsteps, cfl) : tri_batch_t<double, 1, false>(c, nsteps, cfl);
}

// LDS bytes a block size needs (for choosing B and the launch attribute):
// the cell records, then two fluctuation records per edge (TriRec)
template <int NL, int NV> static size_t tri_lds_rec(size_t rs, int lc_max, int e_max)
{
    using R = TriRec<NL, NV>;
    return ((size_t)(R::SA + R::AX) * lc_max + (size_t)2 * R::ER * e_max) * rs;
}
size_t tri_lds_bytes(int nv, size_t rs, int lc_max, int e_max)
{
    return nv == 6 ? tri_lds_rec<2, 6>(rs, lc_max, e_max)
                   : nv == 4 ? tri_lds_rec<1, 4>(rs, lc_max, e_max) : tri_lds_rec<1, 3>(rs, lc_max, e_max);
}

// Reals per edge fluctuation record (the host encodes slots with it).
int tri_edge_rec(int nv) { return nv | 1; }

} // namespace swe
