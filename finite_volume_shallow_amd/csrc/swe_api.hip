// C ABI of the shallow-water step library (see include/swe.h).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "swe_internal.hpp"

using namespace swe;

namespace {

thread_local std::string g_create_err; // detail of the last failed create

struct Fail {
    int code;
};

#define HIPTRY(call)                                                                         \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess) {                                                              \
            c->err = std::string(#call) + ": " + hipGetErrorString(e_);                      \
            throw Fail{SWE_E_HIP};                                                           \
        }                                                                                    \
    } while (0)

void *dev_alloc(swe_ctx *c, size_t bytes)
{
    void *p = nullptr;
    if (bytes == 0) bytes = 8;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
        c->err = std::string("hipMalloc(") + std::to_string(bytes) + "): " + hipGetErrorString(e);
        (void)hipGetLastError();
        throw Fail{e == hipErrorOutOfMemory ? SWE_E_NOMEM : SWE_E_HIP};
    }
    c->allocs.push_back(p);
    return p;
}

// Upload a host double array as the context's real type.
void upload_real(swe_ctx *c, void *dst, const double *src, int64_t n)
{
    if (c->prec == SWE_F64) {
        HIPTRY(hipMemcpyAsync(dst, src, n * sizeof(double), hipMemcpyHostToDevice, c->stream));
        HIPTRY(hipStreamSynchronize(c->stream));
    } else {
        std::vector<float> tmp(n);
        for (int64_t i = 0; i < n; ++i) tmp[i] = (float)src[i];
        HIPTRY(hipMemcpyAsync(dst, tmp.data(), n * sizeof(float), hipMemcpyHostToDevice, c->stream));
        HIPTRY(hipStreamSynchronize(c->stream));
    }
}

void upload_raw(swe_ctx *c, void *dst, const void *src, size_t bytes)
{
    HIPTRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, c->stream));
    HIPTRY(hipStreamSynchronize(c->stream));
}

int validate(const swe_mesh_desc *d, std::string &err)
{
    if (d->abi_version != SWE_ABI_VERSION) { err = "abi_version mismatch"; return SWE_E_INVAL; }
    if (d->nlayers != 1 && d->nlayers != 2) { err = "nlayers must be 1 or 2"; return SWE_E_INVAL; }
    if (d->ntracers != 0 && d->ntracers != 1) { err = "ntracers must be 0 or 1"; return SWE_E_INVAL; }
    if (d->nlayers == 2 && d->ntracers) { err = "a pollutant is supported with one layer only"; return SWE_E_INVAL; }
    if (d->precision != SWE_F64 && d->precision != SWE_F32) { err = "bad precision"; return SWE_E_INVAL; }
    if (d->path < SWE_PATH_AUTO || d->path > SWE_PATH_RECOMPUTE) { err = "bad path"; return SWE_E_INVAL; }
    if (d->scheme != SWE_SCHEME_IR_ROE && d->scheme != SWE_SCHEME_ROE) { err = "bad scheme"; return SWE_E_INVAL; }
    if (d->entropy_fix != SWE_ENTROPY_FIX_NONE && d->entropy_fix != SWE_ENTROPY_FIX_HH) { err = "bad entropy_fix"; return SWE_E_INVAL; }
    if (d->entropy_fix == SWE_ENTROPY_FIX_HH && (d->nlayers != 1 || d->path == SWE_PATH_RECOMPUTE)) {
        err = "the entropy fix is available for one layer on the fused and edge paths";
        return SWE_E_INVAL;
    }
    if (!(d->g > 0.0) || !std::isfinite(d->g)) { err = "g must be > 0"; return SWE_E_INVAL; }
    if (d->nlayers == 2 && !(d->r > 0.0 && d->r < 1.0)) { err = "r must lie in (0, 1)"; return SWE_E_INVAL; }
    if (d->mesh_kind == SWE_MESH_CART) {
        if (d->nlayers != 1) { err = "two layers are supported on triangle meshes only"; return SWE_E_INVAL; }
        if (d->nx < 2 || d->ny < 2) { err = "nx and ny must be >= 2"; return SWE_E_INVAL; }
        if (!(d->dx > 0.0) || !(d->dy > 0.0)) { err = "dx and dy must be > 0"; return SWE_E_INVAL; }
        if ((d->bc_x != SWE_BC_WALL && d->bc_x != SWE_BC_PERIODIC) ||
            (d->bc_y != SWE_BC_WALL && d->bc_y != SWE_BC_PERIODIC)) { err = "bad boundary condition"; return SWE_E_INVAL; }
    } else if (d->mesh_kind == SWE_MESH_TRI) {
        if (!d->node_xy || !d->tri) { err = "node_xy and tri are required"; return SWE_E_INVAL; }
        if (d->nnodes < 3 || d->ncells < 1) { err = "empty triangle mesh"; return SWE_E_INVAL; }
    } else {
        err = "bad mesh_kind";
        return SWE_E_INVAL;
    }
    return SWE_OK;
}

template <typename T> void upload_geometry(swe_ctx *c, const HostEdges &h)
{
    const int64_t E = c->E, N = c->N;
    auto put = [&](const std::vector<double> &src) {
        void *p = dev_alloc(c, E * sizeof(T));
        std::vector<T> tmp(src.begin(), src.end());
        upload_raw(c, p, tmp.data(), E * sizeof(T));
        return p;
    };
    c->e_nx = put(h.nx);
    c->e_ny = put(h.ny);
    c->e_len = put(h.len);
    std::vector<T> ar(N), iar(N);
    for (int64_t i = 0; i < N; ++i) {
        ar[i] = (T)h.area[i];
        iar[i] = (T)(1.0 / h.area[i]);
    }
    c->c_area = dev_alloc(c, N * sizeof(T));
    c->c_iarea = dev_alloc(c, N * sizeof(T));
    upload_raw(c, c->c_area, ar.data(), N * sizeof(T));
    upload_raw(c, c->c_iarea, iar.data(), N * sizeof(T));
}

// Rows per tile of the fused Cartesian kernel (one 64-lane wavefront per
// tile of 60 columns) and whether odd row blocks march downward.  Large
// grids: 20 rows, alternating (measured on 4096^2 with the interleaved
// state: 133.2 us per step against 134.0 at 16 rows, 135.4 at 24 and 138.0
// at 12; the halo rows two neighbouring tiles share are read close together
// and served from L2).  Smaller grids: 10 rows, halved while there are fewer than 1024
// tiles, down to 4.  SWE_CART_TY / SWE_CART_ALT override both (tuning and
// tests).  With periodic y a tile's march (its rows and two halo rows on
// either side) wraps once at most, so a tile has fewer rows than the grid.
static int cart_ty_limit(int64_t ny, bool pery, int ty)
{
    return pery ? (int)std::min<int64_t>(ty, std::max<int64_t>(1, ny - 1)) : ty;
}

void cart_tiling(int64_t nx, int64_t ny, bool pery, int &ty, int &alt)
{
    const int64_t strips = (nx + 59) / 60;
    if (strips * ((ny + 11) / 12) >= 8192) {
        ty = 20;
        alt = 1;
    } else {
        ty = 10;
        while (ty > 4 && strips * ((ny + ty - 1) / ty) < 1024) ty = std::max(4, ty / 2);
        alt = 0;
    }
    if (const char *e = std::getenv("SWE_CART_TY")) { // tuning overrides
        const int v = std::atoi(e);
        if (v >= 4 && v <= 4096) ty = v;
    }
    if (const char *e = std::getenv("SWE_CART_ALT")) alt = std::atoi(e) != 0;
    ty = cart_ty_limit(ny, pery, ty);
}

template <typename T> void upload_blocks(swe_ctx *c, const HostBlocks &hb)
{
    auto ints = [&](const std::vector<int32_t> &v) {
        int32_t *p = (int32_t *)dev_alloc(c, v.size() * sizeof(int32_t));
        upload_raw(c, p, v.data(), v.size() * sizeof(int32_t));
        return p;
    };
    auto reals = [&](const std::vector<double> &v) {
        void *p = dev_alloc(c, v.size() * sizeof(T));
        std::vector<T> tmp(v.begin(), v.end());
        upload_raw(c, p, tmp.data(), v.size() * sizeof(T));
        return p;
    };
    c->tb.B = hb.B;
    c->tb.nblocks = hb.nblocks;
    int upd_max = 0;
    for (int b = 0; b < hb.nblocks; ++b) upd_max = std::max(upd_max, hb.slot_off[b + 1] - hb.slot_off[b]);
    c->tb.rounds = (std::max(std::max(hb.lc_max, hb.e_max), upd_max) + c->tb.nt - 1) / c->tb.nt;
    c->tb.lc_max = hb.lc_max;
    c->tb.e_max = hb.e_max;
    c->tb.halo_off = ints(hb.halo_off);
    c->tb.halo_ids = ints(hb.halo_ids);
    c->tb.n1 = ints(hb.n1);
    c->tb.edge_off = ints(hb.edge_off);
    c->tb.e_s0 = ints(hb.e_s0);
    c->tb.slot_off = ints(hb.slot_off);
    c->tb.e_ab = (uint32_t *)dev_alloc(c, hb.e_ab.size() * sizeof(uint32_t));
    upload_raw(c, c->tb.e_ab, hb.e_ab.data(), hb.e_ab.size() * sizeof(uint32_t));
    c->tb.e_gx = reals(hb.e_gx);
    c->tb.e_gy = reals(hb.e_gy);
    c->tb.iarea = reals(hb.iarea);
    // slots as the kernel addresses its fluctuation records:
    // (side e_max + edge) er, er = reals per record
    const unsigned er = (unsigned)tri_edge_rec(c->nv);
    std::vector<uint16_t> enc(hb.slots.size(), 0);
    for (size_t i = 0; i < hb.slots.size(); ++i)
        if (i % 4 != 3)
            enc[i] = (uint16_t)(((hb.slots[i] & 1u) * (unsigned)hb.e_max + (hb.slots[i] >> 1)) * er);
    c->tb.slots = (uint16_t *)dev_alloc(c, enc.size() * sizeof(uint16_t));
    upload_raw(c, c->tb.slots, enc.data(), enc.size() * sizeof(uint16_t));
    // the pipelined kernel's rows in 4 bytes: three 10-bit record indices
    // side e_max + edge (below 1024: its blocks have at most 512 local
    // edges), which the kernel scales by er itself
    if (c->tb.pipe_wgs != 0) {
        const size_t rows = hb.slots.size() / 4;
        std::vector<uint32_t> enc32(rows, 0u);
        for (size_t r = 0; r < rows; ++r)
            for (int j = 0; j < 3; ++j) {
                const unsigned sl = hb.slots[4 * r + j];
                const unsigned idx = (sl & 1u) * (unsigned)hb.e_max + (sl >> 1);
                if (idx >= 1024u) { // excluded by the one-round check
                    c->err = "triangle block too large for the pipelined kernel's slot rows";
                    throw Fail{SWE_E_INVAL};
                }
                enc32[r] |= idx << (10 * j);
            }
        c->tb.slots32 = (uint32_t *)dev_alloc(c, rows * sizeof(uint32_t));
        upload_raw(c, c->tb.slots32, enc32.data(), rows * sizeof(uint32_t));
    }
}

void free_all(swe_ctx *c)
{
    for (void *p : c->allocs) (void)hipFree(p);
    c->allocs.clear();
    if (c->h_pinned) (void)hipHostFree(c->h_pinned);
    c->h_pinned = nullptr;
    if (c->own_stream && c->stream) (void)hipStreamDestroy(c->stream);
    c->stream = nullptr;
}

// ---- scratch of swe_step_noalloc
// The per-batch bookkeeping of a batch that swe_step_noalloc runs: three
// banks of 64 partial dt minima and the triangle path's block counters
// (PART_DOUBLES), the 8-double step record (dt slots, time, flags, last dt)
// and the dt history of up to SWE_NOALLOC_MAX_STEPS steps, in a file-scope
// device array (about 15.9 KB per GPU, held until the process ends).  Host
// code never passes `scratch` itself to a kernel or a copy: its name is a
// host-side stand-in.  The device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept in g_scratch_dev.
constexpr int NA_PART = PART_DOUBLES;
constexpr int NA_BOOK = 8;
constexpr int NA_DOUBLES = NA_PART + NA_BOOK + SWE_NOALLOC_MAX_STEPS;
static __device__ __align__(256) double scratch[NA_DOUBLES];

std::mutex g_scratch_mu;
std::vector<double *> g_scratch_dev; // per device id; nullptr until taken

// The device address of `scratch` on the current device (cached per device).
hipError_t scratch_address(int device, double **out)
{
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (device < 0) return hipErrorInvalidDevice;
    if ((size_t)device >= g_scratch_dev.size()) g_scratch_dev.resize((size_t)device + 1, nullptr);
    if (!g_scratch_dev[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_dev[device] = static_cast<double *>(p);
    }
    *out = g_scratch_dev[device];
    return hipSuccess;
}

// n doubles from src to dst, ordered on the stream (a kernel rather than a
// memory copy node, so that a captured graph holds kernels only).
__global__ void k_copy_doubles(const double *__restrict__ src, double *__restrict__ dst, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
}

hipError_t copy_doubles(hipStream_t st, const double *src, double *dst, int n)
{
    hipLaunchKernelGGL(k_copy_doubles, dim3(1), dim3(256), 0, st, src, dst, n);
    return hipGetLastError();
}

int status_from_flags(unsigned f)
{
    if (f & FLAG_NONHYPERBOLIC) return SWE_E_NONHYPERBOLIC;
    if (f & FLAG_DEPTH) return SWE_E_DEPTH;
    if (f & FLAG_NONFINITE) return SWE_E_NONFINITE;
    return SWE_OK;
}

} // namespace

extern "C" {

const char *swe_strerror(int s)
{
    switch (s) {
    case SWE_OK: return "ok";
    case SWE_E_INVAL: return "invalid argument or mesh";
    case SWE_E_NOMEM: return "out of memory";
    case SWE_E_HIP: return "HIP runtime error";
    case SWE_E_NOSTATE: return "no state set";
    case SWE_E_DEPTH: return "a layer depth became <= 0";
    case SWE_E_NONFINITE: return "a state value became non-finite";
    case SWE_E_NONHYPERBOLIC: return "two-layer Roe matrix with complex eigenvalues";
    default: return "unknown status";
    }
}

const char *swe_last_error(const swe_ctx *c) { return c ? c->err.c_str() : g_create_err.c_str(); }
int swe_nvars(const swe_ctx *c) { return c ? c->nv : -1; }
int64_t swe_ncells(const swe_ctx *c) { return c ? c->N : -1; }
int swe_path(const swe_ctx *c) { return c ? c->path : -1; }

const char *swe_describe(const swe_ctx *c) { return c ? c->desc.c_str() : ""; }

int swe_create_mesh(const swe_mesh_desc *d, swe_ctx **out)
{
    if (!out) return SWE_E_INVAL;
    *out = nullptr;
    if (!d) return SWE_E_INVAL;
    swe_ctx *c = new (std::nothrow) swe_ctx();
    if (!c) return SWE_E_NOMEM;
    g_create_err.clear();
    int st = validate(d, c->err);
    if (st != SWE_OK) {
        g_create_err = c->err;
        delete c;
        return st;
    }
    try {
        c->kind = d->mesh_kind;
        c->nlayers = d->nlayers;
        c->ntracers = d->ntracers;
        c->prec = d->precision;
        c->classical = d->scheme == SWE_SCHEME_ROE;
        c->hh = d->entropy_fix == SWE_ENTROPY_FIX_HH;
        c->g = d->g;
        c->r = d->nlayers == 2 ? d->r : 0.0;
        c->nx = d->nx;
        c->ny = d->ny;
        c->dx = d->dx;
        c->dy = d->dy;
        c->bc_x = d->bc_x;
        c->bc_y = d->bc_y;
        c->nv = d->nlayers == 2 ? 6 : 3 + d->ntracers;
        c->rs = c->prec == SWE_F32 ? 4 : 8;
        // fused paths: one-layer Cartesian grids and every triangle mesh;
        // SWE_PATH_EDGE forces the explicit-edge path
        const bool fused_ok = d->mesh_kind == SWE_MESH_TRI || d->nlayers == 1;
        if (d->path == SWE_PATH_FUSED && !fused_ok) {
            c->err = "no fused path for this mesh";
            throw Fail{SWE_E_INVAL};
        }
        c->path = (d->path == SWE_PATH_EDGE || !fused_ok) ? SWE_PATH_EDGE : SWE_PATH_FUSED;
        if (d->path == SWE_PATH_RECOMPUTE) {
            if (d->scheme != SWE_SCHEME_IR_ROE) {
                c->err = "the recomputation path exists for the IR-Roe flux only";
                throw Fail{SWE_E_INVAL};
            }
            c->path = SWE_PATH_RECOMPUTE;
        }
        // the fused kernel addresses the state (nv interleaved reals per
        // cell) and the bed with 32-bit byte offsets
        if (d->mesh_kind == SWE_MESH_CART &&
            (d->nx > (int64_t)1 << 30 || d->ny > (int64_t)1 << 30 ||
             (double)d->nx * (double)d->ny * (d->precision == SWE_F32 ? 4 : 8) *
                     (c->path == SWE_PATH_EDGE ? 1 : c->nv) >= 4294967296.0)) {
            c->err = "grid too large";
            throw Fail{SWE_E_INVAL};
        }
        c->interleaved = c->path != SWE_PATH_EDGE; // the fused paths keep per-cell records
        c->N = d->mesh_kind == SWE_MESH_CART ? d->nx * d->ny : d->ncells;

        // host-side mesh work first: mesh errors are reported without
        // touching the GPU
        HostEdges he;
        HostBlocks hb;
        std::vector<int32_t> tri_int;
        if (c->path == SWE_PATH_EDGE) {
            if (d->mesh_kind == SWE_MESH_CART)
                st = build_cart_edges(d->nx, d->ny, d->dx, d->dy, d->bc_x, d->bc_y, he, c->err);
            else
                st = build_tri_edges(d->nnodes, d->node_xy, d->ncells, d->tri, he, c->err);
            if (st != SWE_OK) throw Fail{st};
        } else if (d->mesh_kind == SWE_MESH_TRI) {
            // validate the caller's mesh first (node range, orientation)
            for (int64_t t = 0; t < 3 * d->ncells; ++t)
                if (d->tri[t] < 0 || d->tri[t] >= d->nnodes) {
                    c->err = "node id out of range in triangle " + std::to_string(t / 3);
                    throw Fail{SWE_E_INVAL};
                }
            morton_perm(d->nnodes, d->node_xy, d->ncells, d->tri, c->perm_host);
            tri_int.resize(3 * d->ncells);
            for (int64_t i = 0; i < d->ncells; ++i)
                for (int k = 0; k < 3; ++k) tri_int[3 * i + k] = d->tri[3 * (int64_t)c->perm_host[i] + k];
            st = build_tri_edges(d->nnodes, d->node_xy, d->ncells, tri_int.data(), he, c->err);
            if (st != SWE_OK) throw Fail{st};
            // 512 threads per workgroup.  One layer: blocks of 224 cells,
            // which one round of the threads covers (local cells and edges
            // <= 512), run by the software-pipelined persistent kernel; where
            // a block of the mesh does not fit one round, the size shrinks in
            // steps of 8 cells, down to 192 (the jittered meshes of 1M, 1.28M
            // and 1.5M triangles fit at 216 cells, where the per-block kernel
            // at 288 cells ran 35 % slower per cell); failing that (irregular
            // meshes) 288, 192 or 128 cells with one workgroup per block.
            // Two layers (twice the LDS per cell and edge): 224 cells with one
            // workgroup per block, else 192 or 128.
            // Blocks keep their LDS within 64 KiB (one layer) or 96 KiB (two
            // layers: 224-cell blocks, 79 KiB on the 1M two-layer mesh,
            // measured 2-3 % faster there than 192-cell blocks; 256 cells and
            // more put many edges in a second round of threads, 30-50 %
            // slower).
            c->tb.nt = 512;
            int B = 224;
            bool pipe = c->nv != 6;
            size_t lds_cap = c->nv == 6 ? 98304 : 65536;
            if (const char *e = std::getenv("SWE_TRI_B")) { // tuning overrides
                const int v = std::atoi(e);
                if (v >= 64 && v <= 512 && v % 8 == 0) B = v;
            }
            if (const char *e = std::getenv("SWE_TRI_LDS")) lds_cap = (size_t)std::atol(e);
            if (const char *e = std::getenv("SWE_TRI_NT"))
                if (std::atoi(e) == 256) c->tb.nt = 256;
            if (const char *e = std::getenv("SWE_TRI_PIPE")) pipe = std::atoi(e) != 0;
            if (c->path == SWE_PATH_RECOMPUTE) { // one workgroup of 512 threads per block
                c->tb.nt = 512;
                if (pipe && !std::getenv("SWE_TRI_B")) B = 288; // the per-block kernel's first choice
                pipe = false;
            }
            // Two layers, one workgroup per block: a block whose local
            // cells, edges or updated cells exceed one round of threads
            // makes every block run two rounds (heavier on registers; the
            // classical flux then spills), so the size first shrinks in
            // steps of 8 cells, down to 192, while one block does not fit
            // one round (the 1M two-layer mesh: one of 4,463 blocks of 224
            // cells has 513 local edges, none at 216).
            const bool fit_one_round = c->nv == 6 && !std::getenv("SWE_TRI_B");
            for (;;) {
                st = build_tri_blocks(he, c->N, B, hb, c->err);
                if (st != SWE_OK) throw Fail{st};
                int upd = 0;
                for (int b = 0; b < hb.nblocks; ++b) upd = std::max(upd, hb.slot_off[b + 1] - hb.slot_off[b]);
                const int need = std::max(std::max(hb.lc_max, hb.e_max), upd);
                const bool lds_ok = tri_lds_bytes(c->nv, c->rs, hb.lc_max, hb.e_max) <= lds_cap &&
                                    2 * tri_edge_rec(c->nv) * hb.e_max <= 0xFFFF;
                if (fit_one_round && !pipe && lds_ok && need > c->tb.nt && B > 192 && B <= 224) {
                    B -= 8;
                    continue;
                }
                if (pipe) {
                    if (lds_ok && need <= c->tb.nt) break;
                    if (B > 192 && !std::getenv("SWE_TRI_B")) {
                        B -= 8;
                        continue;
                    }
                    pipe = false; // this mesh: one workgroup per block
                    B = 288;
                    continue;
                }
                const int cap = (c->tb.nt == 256 ? 3 : 2) * c->tb.nt;
                if (lds_ok && need <= cap) break;
                if (B <= 128) {
                    c->err = "triangle blocks do not fit (mesh too irregular); use SWE_PATH_EDGE";
                    throw Fail{SWE_E_INVAL};
                }
                B = B > 192 ? 192 : 128;
            }
            // the fused triangle kernels address these arrays with 32-bit byte offsets
            const uint64_t lim = (uint64_t)1 << 32;
            if (hb.e_ab.size() * 4 > lim || hb.halo_ids.size() * 4 > lim || hb.slots.size() * 2 > lim ||
                hb.e_gx.size() * c->rs > lim || hb.iarea.size() * c->rs > lim ||
                (uint64_t)c->N * c->nv * c->rs > lim) {
                c->err = "triangle mesh too large for the fused path; use SWE_PATH_EDGE";
                throw Fail{SWE_E_INVAL};
            }
            c->tb.pipe_wgs = pipe ? -1 : 0; // -1: size the persistent grid at the first launch
            if (const char *e = std::getenv("SWE_TRI_WGS")) { // tuning override: persistent workgroups
                const int v = std::atoi(e);
                if (pipe && v >= 8) c->tb.pipe_wgs = v; // at least one per XCD
            }
            char buf[256];
            std::snprintf(buf, sizeof buf,
                          "triangle mesh, %s: %s, blocks of %d cells (%d blocks; local cells <= %d, local edges "
                          "<= %d), %d threads per workgroup",
                          c->nv == 6 ? "two layers" : "one layer",
                          pipe ? "software-pipelined persistent kernel" : "one workgroup per block", B, hb.nblocks,
                          hb.lc_max, hb.e_max, c->tb.nt);
            c->desc = buf;
        }

        HIPTRY(hipGetDevice(&c->device));
        // the scratch of swe_step_noalloc on this device (its address is
        // taken here, with the device current, so the call itself needs
        // no set-up)
        HIPTRY(scratch_address(c->device, &c->na_scratch));
        if (d->hip_stream) {
            c->stream = (hipStream_t)d->hip_stream;
        } else {
            HIPTRY(hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking));
            c->own_stream = true;
        }

        if (c->path == SWE_PATH_EDGE) {
            c->E = (int64_t)he.a.size();
            c->e_a = (int32_t *)dev_alloc(c, c->E * sizeof(int32_t));
            c->e_b = (int32_t *)dev_alloc(c, c->E * sizeof(int32_t));
            upload_raw(c, c->e_a, he.a.data(), c->E * sizeof(int32_t));
            upload_raw(c, c->e_b, he.b.data(), c->E * sizeof(int32_t));
            c->c_off = (int32_t *)dev_alloc(c, (c->N + 1) * sizeof(int32_t));
            c->c_edge = (int32_t *)dev_alloc(c, he.ce.size() * sizeof(int32_t));
            upload_raw(c, c->c_off, he.off.data(), (c->N + 1) * sizeof(int32_t));
            upload_raw(c, c->c_edge, he.ce.data(), he.ce.size() * sizeof(int32_t));
            if (c->prec == SWE_F32) upload_geometry<float>(c, he);
            else upload_geometry<double>(c, he);
            c->e_out = dev_alloc(c, (size_t)(2 * c->nv + 1) * c->E * c->rs);
            c->desc = "edge-list path: an edge pass and a cell pass per step, dt by a separate reduction";
        } else if (d->mesh_kind == SWE_MESH_CART) {
            c->cart_part = (double *)dev_alloc(c, PART_DOUBLES * sizeof(double));
            cart_tiling(d->nx, d->ny, d->bc_y == SWE_BC_PERIODIC, c->cart_ty, c->cart_alt);
            // streaming mode (non-temporal state loads, tile order reversed
            // every other step) where the two state copies and the bed exceed
            // the 256 MB last-level cache.  Measured on one box: 4096^2 with
            // a pollutant, float32 (604 MB) 130.6 -> 124.6 us per step,
            // float64 256 -> 247 us; 1024^2 float64 (75 MB) 23.1 -> 24.5 us,
            // so it stays off there.  SWE_CART_STREAM=0/1 overrides the choice.
            c->cart_stream = (double)c->N * c->rs * (2 * c->nv + 1) > 256.0 * (1 << 20);
            if (const char *e = std::getenv("SWE_CART_STREAM")) c->cart_stream = std::atoi(e) != 0;
            char buf[256];
            std::snprintf(buf, sizeof buf,
                          "structured grid %lld x %lld: one fused launch per step, tiles of 60 columns x %d rows%s%s",
                          (long long)d->nx, (long long)d->ny, c->cart_ty,
                          c->cart_alt ? ", odd row blocks marching downward" : "",
                          c->cart_stream ? ", streaming mode (non-temporal state loads, tile order reversed every "
                                           "other step)" : "");
            c->desc = buf;
        } else {
            c->cart_part = (double *)dev_alloc(c, PART_DOUBLES * sizeof(double));
            if (c->prec == SWE_F32) upload_blocks<float>(c, hb);
            else upload_blocks<double>(c, hb);
            c->perm = (int32_t *)dev_alloc(c, c->N * sizeof(int32_t));
            upload_raw(c, c->perm, c->perm_host.data(), c->N * sizeof(int32_t));
        }

        c->desc = std::string(c->classical ? "classical Roe flux" : "IR-Roe flux") +
                  (c->hh ? " with the Harten-Hyman fix" : "") + (c->prec == SWE_F32 ? ", float32" : ", float64") +
                  (c->path == SWE_PATH_RECOMPUTE ? ", every cell evaluating all of its edges" : "") + "; " + c->desc;

        c->state[0] = dev_alloc(c, (size_t)c->nv * c->N * c->rs);
        c->state[1] = dev_alloc(c, (size_t)c->nv * c->N * c->rs);
        c->zbed = dev_alloc(c, (size_t)c->N * c->rs);

        double *bk = (double *)dev_alloc(c, 8 * sizeof(double));
        c->book.slots = bk;
        c->book.t = bk + 3;
        c->book.flags = reinterpret_cast<unsigned *>(bk + 4);
        c->book.last = bk + 5;
        c->hist_cap = 1024;
        c->book.hist = (double *)dev_alloc(c, c->hist_cap * sizeof(double));
        HIPTRY(hipHostMalloc((void **)&c->h_pinned, 8 * sizeof(double), hipHostMallocDefault));
    } catch (const Fail &f) {
        g_create_err = c->err;
        free_all(c);
        delete c;
        return f.code;
    } catch (const std::bad_alloc &) { // host memory for the mesh work
        g_create_err = "out of host memory";
        free_all(c);
        delete c;
        return SWE_E_NOMEM;
    }
    *out = c;
    return SWE_OK;
}

void swe_destroy(swe_ctx *c)
{
    if (!c) return;
    if (c->stream) (void)hipStreamSynchronize(c->stream);
    free_all(c);
    delete c;
}

int swe_set_state(swe_ctx *c, const double *z, const double *const *cons)
{
    if (!c) return SWE_E_INVAL;
    c->dt_ready = false; // a new state: the next batch computes its dt first
    if (!z || !cons) {
        c->err = "NULL argument";
        return SWE_E_INVAL;
    }
    for (int v = 0; v < c->nv; ++v)
        if (!cons[v]) {
            c->err = "NULL state array " + std::to_string(v);
            return SWE_E_INVAL;
        }
    try {
        c->cur = 0;
        std::vector<double> tmp;
        auto ordered = [&](const double *src) -> const double * {
            if (!c->perm) return src;
            tmp.resize(c->N);
            for (int64_t i = 0; i < c->N; ++i) tmp[i] = src[c->perm_host[i]];
            return tmp.data();
        };
        upload_real(c, c->zbed, ordered(z), c->N);
        if (c->interleaved) { // per-cell records (state_offset), internal order
            std::vector<double> rec((size_t)c->nv * c->N);
            for (int64_t i = 0; i < c->N; ++i) {
                const int64_t k = c->perm ? c->perm_host[i] : i;
                for (int v = 0; v < c->nv; ++v) rec[state_offset(c, v, i)] = cons[v][k];
            }
            upload_real(c, c->state[0], rec.data(), (int64_t)c->nv * c->N);
        } else {
            for (int v = 0; v < c->nv; ++v)
                upload_real(c, (char *)c->state[0] + (size_t)v * c->N * c->rs, ordered(cons[v]), c->N);
        }
    } catch (const Fail &f) {
        return f.code;
    } catch (const std::bad_alloc &) {
        c->err = "out of host memory";
        return SWE_E_NOMEM;
    }
    c->has_state = true;
    c->err.clear();
    return SWE_OK;
}

int swe_set_state_device(swe_ctx *c, const void *z, const void *const *cons)
{
    if (!c) return SWE_E_INVAL;
    c->dt_ready = false;
    if (!z || !cons) {
        c->err = "NULL argument";
        return SWE_E_INVAL;
    }
    for (int v = 0; v < c->nv; ++v)
        if (!cons[v]) {
            c->err = "NULL state array " + std::to_string(v);
            return SWE_E_INVAL;
        }
    try {
        c->cur = 0;
        const size_t bytes = (size_t)c->N * c->rs;
        if (c->perm) { // fused triangle path: records in internal order
            HIPTRY(launch_permute(c, z, c->zbed, 1));
            HIPTRY(launch_tri_pack(c, cons, c->state[0], 1));
        } else {
            HIPTRY(hipMemcpyAsync(c->zbed, z, bytes, hipMemcpyDeviceToDevice, c->stream));
            if (c->interleaved) {
                HIPTRY(launch_cart_pack(c, cons, c->state[0], 1));
            } else {
                for (int v = 0; v < c->nv; ++v)
                    HIPTRY(hipMemcpyAsync((char *)c->state[0] + v * bytes, cons[v], bytes, hipMemcpyDeviceToDevice,
                                          c->stream));
            }
        }
    } catch (const Fail &f) {
        return f.code;
    } catch (const std::bad_alloc &) {
        c->err = "out of host memory";
        return SWE_E_NOMEM;
    }
    c->has_state = true;
    c->err.clear();
    return SWE_OK;
}

} // extern "C"

namespace {

// The batch of swe_step and swe_step_noalloc.  With `na`, the batch's
// bookkeeping lives in the scratch array instead of the context's own
// buffers: the context's partial-minimum banks (dt of the current state,
// fused paths) are copied in first, and the banks and the dt history are
// copied back afterwards, so the context continues exactly as after
// swe_step; nothing is allocated.
int run_batch(swe_ctx *c, int32_t nsteps, double cfl, double *t_adv, double *last_dt, bool na)
{
    if (nsteps < 0 || !(cfl > 0.0 && cfl <= 1.0)) {
        c->err = "nsteps must be >= 0 and cfl in (0, 1]";
        return SWE_E_INVAL;
    }
    if (na && nsteps > SWE_NOALLOC_MAX_STEPS) {
        c->err = "swe_step_noalloc takes at most " + std::to_string(SWE_NOALLOC_MAX_STEPS) + " steps per call";
        return SWE_E_INVAL;
    }
    if (!c->has_state) {
        c->err = "swe_step before swe_set_state";
        return SWE_E_NOSTATE;
    }
    if (t_adv) *t_adv = 0.0;
    if (last_dt) *last_dt = 0.0;
    c->hist_count = 0;
    if (nsteps == 0) return SWE_OK;
    unsigned flags = 0;
    const StepBook own_book = c->book;
    double *const own_part = c->cart_part;
    const bool fused = c->path != SWE_PATH_EDGE;
    try {
        if (!na && nsteps > c->hist_cap) {
            int64_t cap = c->hist_cap;
            while (cap < nsteps) cap *= 2;
            HIPTRY(hipStreamSynchronize(c->stream));
            void *old = c->book.hist;
            c->book.hist = (double *)dev_alloc(c, cap * sizeof(double));
            for (auto &p : c->allocs)
                if (p == old) {
                    (void)hipFree(old);
                    p = c->allocs.back();
                    c->allocs.pop_back();
                    break;
                }
            c->hist_cap = cap;
        }
        if (na) {
            double *sp = c->na_scratch, *sb = sp + NA_PART;
            if (fused) HIPTRY(copy_doubles(c->stream, own_part, sp, NA_PART));
            c->book = StepBook{sb, sb + 3, reinterpret_cast<unsigned *>(sb + 4), sb + 5, sb + NA_BOOK};
            if (fused) c->cart_part = sp;
        }
        if (fused) { // fused (or its recomputation variant)
            if (c->kind == SWE_MESH_CART) HIPTRY(launch_cart_batch(c, nsteps, cfl));
            else HIPTRY(launch_tri_batch(c, nsteps, cfl));
            c->cur ^= (nsteps & 1); // ping-pong: the last launch wrote the other buffer
            // the last launch left dt of the new state in the next bank: a
            // following batch with the same cfl starts from it
            c->bank0 = (int)((c->bank0 + nsteps) % 3);
            c->dt_ready = true;
            c->dt_cfl = cfl;
        } else {
            HIPTRY(launch_batch_init(c));
            for (int64_t s = 0; s < nsteps; ++s) HIPTRY(launch_edge_step(c, s, cfl));
        }
        if (na) { // the banks and the history back into the context
            if (fused) HIPTRY(copy_doubles(c->stream, c->cart_part, own_part, NA_PART));
            HIPTRY(copy_doubles(c->stream, c->book.hist, own_book.hist, nsteps));
        }
        // slots, t, flags and the last dt in one copy
        HIPTRY(hipMemcpyAsync(c->h_pinned, c->book.slots, 8 * sizeof(double), hipMemcpyDeviceToHost, c->stream));
        HIPTRY(hipStreamSynchronize(c->stream));
        std::memcpy(&flags, c->h_pinned + 4, sizeof(unsigned));
    } catch (const Fail &f) {
        c->book = own_book;
        c->cart_part = own_part;
        c->dt_ready = false;
        return f.code;
    } catch (const std::bad_alloc &) {
        c->book = own_book;
        c->cart_part = own_part;
        c->err = "out of host memory";
        return SWE_E_NOMEM;
    }
    c->book = own_book;
    c->cart_part = own_part;
    c->hist_count = nsteps;
    if (t_adv) *t_adv = c->h_pinned[3];
    if (last_dt) *last_dt = c->h_pinned[5];
    const int st = status_from_flags(flags);
    if (st != SWE_OK) {
        c->err = swe_strerror(st);
        c->dt_ready = false;
    }
    return st;
}

} // namespace

extern "C" {

int swe_step(swe_ctx *c, int32_t nsteps, double cfl, double *t_adv, double *last_dt)
{
    if (!c) return SWE_E_INVAL;
    return run_batch(c, nsteps, cfl, t_adv, last_dt, false);
}

int swe_step_noalloc(swe_ctx *c, int32_t nsteps, double cfl, double *t_adv, double *last_dt)
{
    if (!c) return SWE_E_INVAL;
    return run_batch(c, nsteps, cfl, t_adv, last_dt, true);
}

int swe_get_state(swe_ctx *c, double *const *out)
{
    if (!c) return SWE_E_INVAL;
    if (!out) {
        c->err = "NULL argument";
        return SWE_E_INVAL;
    }
    for (int v = 0; v < c->nv; ++v)
        if (!out[v]) {
            c->err = "NULL output array " + std::to_string(v);
            return SWE_E_INVAL;
        }
    if (!c->has_state) {
        c->err = "swe_get_state before swe_set_state";
        return SWE_E_NOSTATE;
    }
    try {
        const char *base = (const char *)c->state[c->cur];
        std::vector<double> d64;
        std::vector<float> f32;
        if (c->interleaved) { // per-cell records (state_offset), internal order
            const size_t n = (size_t)c->nv * c->N;
            d64.resize(n);
            if (c->prec == SWE_F64) {
                HIPTRY(hipMemcpyAsync(d64.data(), base, n * 8, hipMemcpyDeviceToHost, c->stream));
                HIPTRY(hipStreamSynchronize(c->stream));
            } else {
                f32.resize(n);
                HIPTRY(hipMemcpyAsync(f32.data(), base, n * 4, hipMemcpyDeviceToHost, c->stream));
                HIPTRY(hipStreamSynchronize(c->stream));
                for (size_t i = 0; i < n; ++i) d64[i] = f32[i];
            }
            for (int64_t i = 0; i < c->N; ++i) {
                const int64_t k = c->perm ? c->perm_host[i] : i;
                for (int v = 0; v < c->nv; ++v) out[v][k] = d64[state_offset(c, v, i)];
            }
            return SWE_OK;
        }
        for (int v = 0; v < c->nv; ++v) {
            const double *src;
            if (c->prec == SWE_F64) {
                d64.resize(c->N);
                HIPTRY(hipMemcpyAsync(d64.data(), base + (size_t)v * c->N * 8, c->N * 8, hipMemcpyDeviceToHost,
                                      c->stream));
                HIPTRY(hipStreamSynchronize(c->stream));
                src = d64.data();
            } else {
                f32.resize(c->N);
                d64.resize(c->N);
                HIPTRY(hipMemcpyAsync(f32.data(), base + (size_t)v * c->N * 4, c->N * 4, hipMemcpyDeviceToHost,
                                      c->stream));
                HIPTRY(hipStreamSynchronize(c->stream));
                for (int64_t i = 0; i < c->N; ++i) d64[i] = f32[i];
                src = d64.data();
            }
            if (c->perm)
                for (int64_t i = 0; i < c->N; ++i) out[v][c->perm_host[i]] = src[i];
            else
                std::memcpy(out[v], src, c->N * sizeof(double));
        }
    } catch (const Fail &f) {
        return f.code;
    } catch (const std::bad_alloc &) {
        c->err = "out of host memory";
        return SWE_E_NOMEM;
    }
    return SWE_OK;
}

int swe_get_state_device(swe_ctx *c, void *const *out)
{
    if (!c) return SWE_E_INVAL;
    if (!out) {
        c->err = "NULL argument";
        return SWE_E_INVAL;
    }
    for (int v = 0; v < c->nv; ++v)
        if (!out[v]) {
            c->err = "NULL output array " + std::to_string(v);
            return SWE_E_INVAL;
        }
    if (!c->has_state) {
        c->err = "swe_get_state before swe_set_state";
        return SWE_E_NOSTATE;
    }
    try {
        const size_t bytes = (size_t)c->N * c->rs;
        if (c->interleaved) {
            if (c->perm) HIPTRY(launch_tri_pack(c, (const void *const *)out, c->state[c->cur], 0));
            else HIPTRY(launch_cart_pack(c, (const void *const *)out, c->state[c->cur], 0));
            return SWE_OK;
        }
        for (int v = 0; v < c->nv; ++v) {
            const char *src = (const char *)c->state[c->cur] + v * bytes;
            if (c->perm) HIPTRY(launch_permute(c, src, out[v], 0));
            else HIPTRY(hipMemcpyAsync(out[v], src, bytes, hipMemcpyDeviceToDevice, c->stream));
        }
    } catch (const Fail &f) {
        return f.code;
    } catch (const std::bad_alloc &) {
        c->err = "out of host memory";
        return SWE_E_NOMEM;
    }
    return SWE_OK;
}

int swe_get_dt_history(swe_ctx *c, double *out, int64_t cap, int64_t *count)
{
    if (!c) return SWE_E_INVAL;
    if (!count || cap < 0 || (cap > 0 && !out)) {
        c->err = "bad arguments";
        return SWE_E_INVAL;
    }
    *count = c->hist_count;
    const int64_t n = cap < c->hist_count ? cap : c->hist_count;
    if (n == 0) return SWE_OK;
    try {
        HIPTRY(hipMemcpyAsync(out, c->book.hist, n * sizeof(double), hipMemcpyDeviceToHost, c->stream));
        HIPTRY(hipStreamSynchronize(c->stream));
    } catch (const Fail &f) {
        return f.code;
    } catch (const std::bad_alloc &) {
        c->err = "out of host memory";
        return SWE_E_NOMEM;
    }
    return SWE_OK;
}

} // extern "C"
