// Generic explicit-edge-list path (any mesh): three kernels per step.
//
//   k_edge_flux  one thread per edge: gathers the two cells' states
//                (structure-of-arrays, one array per variable), rotates them
//                into the edge frame ([IR] Eq. (2), step 1), evaluates the
//                Roe flux fluctuations for both sides and the edge's largest
//                wave speed, rotates back (step 4) and writes
//                |G| T^-1 (fluctuation) for each side plus |G| ||D||_inf.
//   k_cell_dt    grid-stride over the cells: sums |G| ||D||_inf over each
//                cell's edges and forms dt_i = 2 gamma |V_i| / sum ([IR]
//                Eq. (5)); a wavefront min, a block min and one atomic min
//                per block on the bit pattern of the (non-negative) double.
//                At most DT_BLOCKS blocks, so that the atomics on the one
//                dt slot stay few.
//   k_cell_update one thread per cell: gathers its edges' fluctuations in a
//                fixed order (no atomics, deterministic) and applies Eq. (4)
//                with the global dt.
#include <algorithm>

#include "dt_reduce.hpp"
#include "roe_device.hpp"
#include "swe_internal.hpp"

namespace swe {

template <typename T> struct EdgeArrays {
    const int32_t *a, *b;
    const T *nx, *ny, *len;
};

// FX: the flux variant (FLUX_IR, FLUX_ROE, FLUX_IR_HH).
template <typename T, int NL, bool TR, int FX>
__global__ __launch_bounds__(256) void k_edge_flux(int64_t E, EdgeArrays<T> ed, StatePtrs<T> W,
                                                   const T *__restrict__ z, T g, T r,
                                                   T *__restrict__ out, unsigned *flags)
{
    constexpr int NV = NL == 2 ? 6 : (TR ? 4 : 3);
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const int32_t a = ed.a[e], b = ed.b[e];
    const T nx = ed.nx[e], ny = ed.ny[e], len = ed.len[e];
    T A[NV], B[NV], speed;
    if constexpr (NL == 1) {
        const T ha = W.v[0][a], qxa = W.v[1][a], qya = W.v[2][a];
        const T ca = TR ? W.v[3][a] : T(0);
        const T qna = qxa * nx + qya * ny, qta = -qxa * ny + qya * nx;
        Flux1<T, TR> f;
        if (b >= 0) {
            const T hb = W.v[0][b], qxb = W.v[1][b], qyb = W.v[2][b];
            const T cb = TR ? W.v[3][b] : T(0);
            const T qnb = qxb * nx + qyb * ny, qtb = -qxb * ny + qyb * nx;
            f = roe1_interior<T, TR, FX>(ha, qna, qta, ca, z[a], hb, qnb, qtb, cb, z[b], g);
        } else {
            f = roe1_wall<T, TR>(ha, qna, qta, ca, g);
        }
        A[0] = len * f.am;
        A[1] = len * (f.an * nx - f.at * ny);
        A[2] = len * (f.an * ny + f.at * nx);
        B[0] = len * f.bm;
        B[1] = len * (f.bn * nx - f.bt * ny);
        B[2] = len * (f.bn * ny + f.bt * nx);
        if constexpr (TR) {
            A[3] = len * f.ac;
            B[3] = len * f.bc;
        }
        speed = f.speed;
    } else {
        T L[6], R[6];
#pragma unroll
        for (int l = 0; l < 2; ++l) {
            const T qx = W.v[3 * l + 1][a], qy = W.v[3 * l + 2][a];
            L[3 * l] = W.v[3 * l][a];
            L[3 * l + 1] = qx * nx + qy * ny;
            L[3 * l + 2] = -qx * ny + qy * nx;
        }
        Flux2<T> f;
        if (b >= 0) {
#pragma unroll
            for (int l = 0; l < 2; ++l) {
                const T qx = W.v[3 * l + 1][b], qy = W.v[3 * l + 2][b];
                R[3 * l] = W.v[3 * l][b];
                R[3 * l + 1] = qx * nx + qy * ny;
                R[3 * l + 2] = -qx * ny + qy * nx;
            }
            f = roe2_interior<T, flux_classical(FX)>(L, z[a], R, z[b], g, r);
        } else {
            f = roe2_wall<T>(L, z[a], g, r);
        }
        if (f.nonhyp) atomicOr(flags, FLAG_NONHYPERBOLIC);
#pragma unroll
        for (int l = 0; l < 2; ++l) {
            A[3 * l] = len * f.a[3 * l];
            A[3 * l + 1] = len * (f.a[3 * l + 1] * nx - f.a[3 * l + 2] * ny);
            A[3 * l + 2] = len * (f.a[3 * l + 1] * ny + f.a[3 * l + 2] * nx);
            B[3 * l] = len * f.b[3 * l];
            B[3 * l + 1] = len * (f.b[3 * l + 1] * nx - f.b[3 * l + 2] * ny);
            B[3 * l + 2] = len * (f.b[3 * l + 1] * ny + f.b[3 * l + 2] * nx);
        }
        speed = f.speed;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        out[(int64_t)v * E + e] = A[v];
        out[(int64_t)(NV + v) * E + e] = B[v];
    }
    out[(int64_t)(2 * NV) * E + e] = len * speed;
}

// Blocks of k_cell_dt at most: every block ends in one atomic min on the
// same address, and one per 256 cells serialised them (65,536 per step on a
// 4096^2 grid).
constexpr int64_t DT_BLOCKS = 1024;

template <typename T, int NV>
__global__ __launch_bounds__(256) void k_cell_dt(int64_t N, int64_t E, const int32_t *__restrict__ off,
                                                 const int32_t *__restrict__ ce, const T *__restrict__ area,
                                                 const T *__restrict__ out, T cfl, double *slot)
{
    const T *sp = out + (int64_t)(2 * NV) * E;
    double dti = __builtin_inf();
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < N; c += (int64_t)gridDim.x * blockDim.x) {
        T S = T(0);
        for (int32_t k = off[c]; k < off[c + 1]; ++k) S += sp[ce[k] >> 1];
        dti = fmin(dti, (double)(T(2) * cfl * area[c] / S));
    }
    block_min_to_slot(dti, slot);
}

template <typename T, int NV>
__global__ __launch_bounds__(256) void k_cell_update(int64_t N, int64_t E, const int32_t *__restrict__ off,
                                                     const int32_t *__restrict__ ce,
                                                     const T *__restrict__ iarea, const T *__restrict__ out,
                                                     StatePtrs<T> W, StepBook book, int64_t step,
                                                     int nlayers)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int s = (int)(step % 3);
    const double dtd = book.slots[s];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        book.slots[(s + 1) % 3] = __builtin_inf();
        book.hist[step] = dtd;
        book.last[0] = dtd;
        book.t[0] += dtd;
    }
    if (c >= N) return;
    T acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = T(0);
    for (int32_t k = off[c]; k < off[c + 1]; ++k) {
        const int32_t code = ce[k];
        const int64_t e = code >> 1;
        const int side = code & 1;
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] += out[(int64_t)(side * NV + v) * E + e];
    }
    const T f = (T)dtd * iarea[c];
    bool bad_depth = false, bad_val = false;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const T nv = W.v[v][c] - f * acc[v];
        W.v[v][c] = nv;
        bad_val |= !isfinite(nv);
    }
    bad_depth = !(W.v[0][c] > T(0));
    if (nlayers == 2) bad_depth |= !(W.v[3][c] > T(0));
    if (bad_depth) atomicOr(book.flags, FLAG_DEPTH);
    if (bad_val) atomicOr(book.flags, FLAG_NONFINITE);
}

__global__ void k_batch_init(StepBook book)
{
    if (threadIdx.x == 0) {
        book.slots[0] = __builtin_inf();
        book.slots[1] = __builtin_inf();
        book.slots[2] = __builtin_inf();
        book.t[0] = 0.0;
        book.flags[0] = 0u;
    }
}

hipError_t launch_batch_init(swe_ctx *c)
{
    hipLaunchKernelGGL(k_batch_init, dim3(1), dim3(64), 0, c->stream, c->book);
    return hipGetLastError();
}

template <typename T> static StatePtrs<T> state_ptrs(swe_ctx *c)
{
    StatePtrs<T> p;
    for (int v = 0; v < 6; ++v)
        p.v[v] = v < c->nv ? reinterpret_cast<T *>(c->state[c->cur]) + (int64_t)v * c->N : nullptr;
    return p;
}

template <typename T, int NL, bool TR, int FX = FLUX_IR>
static hipError_t edge_step_t(swe_ctx *c, int64_t step, double cfl)
{
    constexpr int NV = NL == 2 ? 6 : (TR ? 4 : 3);
    const int bs = 256;
    EdgeArrays<T> ed{c->e_a, c->e_b, (const T *)c->e_nx, (const T *)c->e_ny, (const T *)c->e_len};
    StatePtrs<T> W = state_ptrs<T>(c);
    T *out = (T *)c->e_out;
    const dim3 ge((unsigned)((c->E + bs - 1) / bs)), gc((unsigned)((c->N + bs - 1) / bs));
    const dim3 gd((unsigned)std::min<int64_t>((c->N + bs - 1) / bs, DT_BLOCKS));
    hipLaunchKernelGGL((k_edge_flux<T, NL, TR, FX>), ge, dim3(bs), 0, c->stream, c->E, ed, W,
                       (const T *)c->zbed, (T)c->g, (T)c->r, out, c->book.flags);
    hipLaunchKernelGGL((k_cell_dt<T, NV>), gd, dim3(bs), 0, c->stream, c->N, c->E, c->c_off, c->c_edge,
                       (const T *)c->c_area, (const T *)out, (T)cfl, c->book.slots + (step % 3));
    hipLaunchKernelGGL((k_cell_update<T, NV>), gc, dim3(bs), 0, c->stream, c->N, c->E, c->c_off,
                       c->c_edge, (const T *)c->c_iarea, (const T *)out, W, c->book, step, c->nlayers);
    return hipGetLastError();
}

template <int FX> static hipError_t edge_step_fx(swe_ctx *c, int64_t step, double cfl)
{
    const bool f32 = c->prec == SWE_F32;
    if (c->nlayers == 2) return f32 ? edge_step_t<float, 2, false, FX>(c, step, cfl) : edge_step_t<double, 2, false, FX>(c, step, cfl);
    if (c->ntracers) return f32 ? edge_step_t<float, 1, true, FX>(c, step, cfl) : edge_step_t<double, 1, true, FX>(c, step, cfl);
    return f32 ? edge_step_t<float, 1, false, FX>(c, step, cfl) : edge_step_t<double, 1, false, FX>(c, step, cfl);
}

hipError_t launch_edge_step(swe_ctx *c, int64_t step, double cfl)
{
    // the entropy fix is one-layer only (checked at create)
    if (c->classical) return c->hh ? edge_step_fx<FLUX_ROE_HH>(c, step, cfl) : edge_step_fx<FLUX_ROE>(c, step, cfl);
    if (c->hh) return edge_step_fx<FLUX_IR_HH>(c, step, cfl);
    return edge_step_fx<FLUX_IR>(c, step, cfl);
}

} // namespace swe
