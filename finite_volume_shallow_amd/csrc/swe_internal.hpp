// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/swe.h"

namespace swe {

// The fused paths' per-batch device bookkeeping, in doubles: three banks of
// 64 partial dt minima, then three banks of eight 32-bit block counters (the
// pipelined triangle kernel's dynamic block schedule, one per XCD band), each
// counter on a 256-byte line of its own: atomics of all eight bands on one
// line serialised and made the triangle step 75 % slower.
constexpr int PART_DOUBLES = 3 * 64 + 3 * 8 * 32;

// Device error flags, OR-ed by the kernels and read once per batch.
enum : unsigned { FLAG_DEPTH = 1u, FLAG_NONFINITE = 2u, FLAG_NONHYPERBOLIC = 4u };

// Host-side explicit edge list with geometry ([IR] Sec. 2.2 notation: edge
// G_ij between cells a = i and b = j, unit normal eta pointing from a to b,
// length |G_ij|; b = -1 marks a reflective wall, eta then points outward).
struct HostEdges {
    std::vector<int32_t> a, b;
    std::vector<double> nx, ny, len;
    std::vector<int32_t> off; // cell -> [off[c], off[c+1]) in ce
    std::vector<int32_t> ce;  // (edge << 1) | side, side 0 = a, 1 = b
    std::vector<double> area;
};

// Per-block data of the fused triangle path.  Cells are taken in blocks of
// B consecutive (Morton-ordered) cells; a block also reads two rings of
// neighbours ("halo"): ring 1 = neighbours of the block, ring 2 = neighbours
// of ring 1.  Its local edges are every edge touching the block or ring 1,
// the ones touching the block first.  Local cell ids: block cells 0..B0-1,
// then ring 1, then ring 2.
struct HostBlocks {
    int B = 0, nblocks = 0;
    int lc_max = 0, e_max = 0;              // largest local cell / edge counts
    std::vector<int32_t> halo_off, halo_ids; // global ids of ring 1 then ring 2 (one padding entry at the end)
    std::vector<int32_t> n1;                 // ring-1 size per block
    std::vector<int32_t> edge_off, e_s0;     // local edges; leading edges touching the block
    std::vector<uint32_t> e_ab;              // local a | local b << 16 (b = 0xFFFF: wall)
    std::vector<double> e_gx, e_gy;          // |G| eta: length times unit normal
    std::vector<int32_t> slot_off;           // per block: first slot row (block + ring 1 cells)
    std::vector<uint16_t> slots;             // 4 per cell: 3 x (local edge << 1 | side), padding
    std::vector<double> iarea;               // 1/|V| per slot row
};

int build_tri_blocks(const HostEdges &he, int64_t ncells, int B, HostBlocks &out, std::string &err);

// Morton order of the triangle centroids (stable): perm[internal] = caller id.
void morton_perm(int64_t nnodes, const double *xy, int64_t ncells, const int32_t *tri,
                 std::vector<int32_t> &perm);

int build_cart_edges(int64_t nx, int64_t ny, double dx, double dy, int bcx, int bcy,
                     HostEdges &out, std::string &err);
int build_tri_edges(int64_t nnodes, const double *xy, int64_t ncells, const int32_t *tri,
                    HostEdges &out, std::string &err);

// Pointer bundle of the state arrays (SoA, one array per variable).
template <typename T> struct StatePtrs {
    T *v[6];
};

// Per-batch bookkeeping on the device: three dt slots used round-robin,
// the accumulated time, error flags, the dt of the latest step and the dt
// history of the batch.  slots, t, flags and last lie in one 8-double
// record (slots[0..2], t, flags, last) that the host reads back in one copy.
struct StepBook {
    double *slots;   // [3], non-negative doubles compared as uint64 bits
    double *t;       // [1]
    unsigned *flags; // [1]
    double *last;    // [1]
    double *hist;    // [hist_cap]
};

} // namespace swe

struct swe_ctx {
    // configuration
    int kind = 0, nlayers = 1, ntracers = 0, prec = SWE_F64, path = SWE_PATH_EDGE;
    double g = 9.81, r = 0.0;
    int64_t nx = 0, ny = 0;
    double dx = 0, dy = 0;
    int bc_x = 0, bc_y = 0;
    int64_t N = 0;
    int nv = 3;
    bool classical = false; // classical Roe flux instead of IR-Roe
    bool hh = false;        // Harten-Hyman entropy fix (one layer)
    size_t rs = 8; // bytes per real
    int device = 0;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    std::string err;
    std::string desc; // what swe_describe returns
    bool has_state = false;

    // state: two copies (ping-pong) of nv * N reals each: nv arrays of N
    // reals (edge path), or interleaved per cell (`interleaved`: record
    // planes on the fused structured path, records of nv reals on the fused
    // triangle path); state_offset addresses all three
    void *state[2] = {nullptr, nullptr};
    bool interleaved = false;
    int cur = 0;
    void *zbed = nullptr;

    // generic edge path
    int64_t E = 0;
    int32_t *e_a = nullptr, *e_b = nullptr;
    void *e_nx = nullptr, *e_ny = nullptr, *e_len = nullptr;
    int32_t *c_off = nullptr, *c_edge = nullptr;
    void *c_area = nullptr, *c_iarea = nullptr;
    void *e_out = nullptr; // (2 nv + 1) * E reals

    // fused Cartesian path
    // fused paths: dt of the current state is already in the partial-minimum
    // bank bank0 when dt_ready (left by the previous batch, for cfl dt_cfl)
    bool dt_ready = false;
    int bank0 = 0;
    double dt_cfl = 0.0;
    int cart_ty = 64;            // rows per tile
    int cart_alt = 0;            // odd row blocks of tiles march downward
    int cart_stream = 0;         // streaming mode: non-temporal state loads, alternating tile order
    double *cart_part = nullptr; // PART_DOUBLES: [3][64] partial dt minima (both fused paths), then the
                                 // triangle path's [3][8] 32-bit block counters

    // fused triangle path: cells in internal (Morton) order
    int32_t *perm = nullptr;          // device: internal index -> caller index
    std::vector<int32_t> perm_host;   // same on the host
    struct {
        int B = 0, nblocks = 0, lc_max = 0, e_max = 0;
        int nt = 512;   // threads per workgroup (256 or 512)
        int rounds = 1; // ceil(max(local cells, local edges, updated cells) / nt), <= 3
        int pipe_wgs = 0; // persistent pipelined workgroups (0: one workgroup per block, -1: not sized yet)
        int32_t *halo_off = nullptr, *halo_ids = nullptr, *n1 = nullptr, *edge_off = nullptr,
                *e_s0 = nullptr, *slot_off = nullptr;
        uint32_t *e_ab = nullptr;
        void *e_gx = nullptr, *e_gy = nullptr, *iarea = nullptr;
        uint16_t *slots = nullptr;
        uint32_t *slots32 = nullptr; // pipelined kernel: three 10-bit record indices per cell
    } tb;

    // step bookkeeping
    swe::StepBook book{nullptr, nullptr, nullptr, nullptr, nullptr};
    int64_t hist_cap = 0, hist_count = 0;
    double *h_pinned = nullptr; // t, last dt, flags
    double *na_scratch = nullptr; // device address of swe_step_noalloc's scratch on this device

    std::vector<void *> allocs; // every device allocation, freed on destroy
};

namespace swe {

// Kernel launchers (kern_*.hip).  Each returns hipSuccess or the launch error.
hipError_t launch_batch_init(swe_ctx *c);
hipError_t launch_edge_step(swe_ctx *c, int64_t step, double cfl);
hipError_t launch_cart_batch(swe_ctx *c, int32_t nsteps, double cfl);
hipError_t launch_tri_batch(swe_ctx *c, int32_t nsteps, double cfl);
hipError_t launch_permute(swe_ctx *c, const void *src, void *dst, int to_internal);
// Structured fused path: pack = 1 interleaves the nv device arrays soa[] into
// the record planes at rec (cart_plane); pack = 0 splits them.
hipError_t launch_cart_pack(swe_ctx *c, const void *const *soa, void *rec, int pack);

// Fused triangle path: pack = 1 moves the nv device arrays soa[] (caller
// cell order) into the per-cell records at rec (internal order); pack = 0
// moves them back.
hipError_t launch_tri_pack(swe_ctx *c, const void *const *soa, void *rec, int pack);

// Record planes of the structured fused path: float32, one plane of nv
// reals per cell; float64, plane 0 holds (h, qx) and plane 1 the remaining
// nv - 2 reals per cell.  Offset, in reals from the state's start, of
// variable v of cell k, and the start of plane 1.
inline int64_t cart_plane1(const swe_ctx *c);
inline int64_t cart_plane_offset(const swe_ctx *c, int v, int64_t k);
// Offset, in reals from the state's start, of variable v of (internal) cell
// k in any path's layout: record planes (structured fused path), records of
// nv reals (fused triangle path) or one array per variable (edge path).
inline int64_t state_offset(const swe_ctx *c, int v, int64_t k);
size_t tri_lds_bytes(int nv, size_t rs, int lc_max, int e_max);
int tri_edge_rec(int nv);

} // namespace swe

inline int64_t swe::cart_plane1(const swe_ctx *c) { return c->rs == 4 ? 0 : 2 * c->N; }
inline int64_t swe::cart_plane_offset(const swe_ctx *c, int v, int64_t k)
{
    if (c->rs == 4) return k * c->nv + v;
    return v < 2 ? 2 * k + v : 2 * c->N + k * (c->nv - 2) + (v - 2);
}
inline int64_t swe::state_offset(const swe_ctx *c, int v, int64_t k)
{
    if (!c->interleaved) return v * c->N + k;
    if (c->kind == SWE_MESH_CART) return cart_plane_offset(c, v, k);
    return k * c->nv + v;
}
