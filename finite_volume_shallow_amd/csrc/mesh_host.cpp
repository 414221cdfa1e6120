// Host-side mesh preprocessing: explicit edge lists with their geometry.
//
// [IR] Sec. 2.2 (de la Asuncion et al.): cells V_i with area |V_i|, edges
// G_ij of length |G_ij| with the unit normal eta_ij pointing from V_i to
// V_j.  Triangles are given counter-clockwise, so the edge from corner k to
// corner k+1 with direction (dx, dy) has outward normal (dy, -dx)/|G|.
#include <algorithm>
#include <cmath>

#include "swe_internal.hpp"

namespace swe {

static void finish_cells(int64_t ncells, HostEdges &out)
{
    const int64_t E = (int64_t)out.a.size();
    out.off.assign(ncells + 1, 0);
    for (int64_t e = 0; e < E; ++e) {
        out.off[out.a[e] + 1]++;
        if (out.b[e] >= 0) out.off[out.b[e] + 1]++;
    }
    for (int64_t c = 0; c < ncells; ++c) out.off[c + 1] += out.off[c];
    out.ce.assign(out.off[ncells], 0);
    std::vector<int32_t> fill(out.off.begin(), out.off.end() - 1);
    for (int64_t e = 0; e < E; ++e) {
        out.ce[fill[out.a[e]]++] = (int32_t)(e << 1);
        if (out.b[e] >= 0) out.ce[fill[out.b[e]]++] = (int32_t)((e << 1) | 1);
    }
}

int build_cart_edges(int64_t nx, int64_t ny, double dx, double dy, int bcx, int bcy,
                     HostEdges &out, std::string &err)
{
    const int64_t N = nx * ny;
    if (N > (int64_t(1) << 30)) {
        err = "grid too large for 32-bit edge indices";
        return SWE_E_INVAL;
    }
    out = HostEdges();
    auto push = [&](int64_t a, int64_t b, double ex, double ey, double len) {
        out.a.push_back((int32_t)a);
        out.b.push_back((int32_t)b);
        out.nx.push_back(ex);
        out.ny.push_back(ey);
        out.len.push_back(len);
    };
    // edges in row-major order of their owner cell: left wall, right
    // neighbour (or wall / periodic wrap), bottom wall, top neighbour
    for (int64_t j = 0; j < ny; ++j)
        for (int64_t i = 0; i < nx; ++i) {
            const int64_t k = j * nx + i;
            if (i == 0 && bcx == SWE_BC_WALL) push(k, -1, -1.0, 0.0, dy);
            if (i + 1 < nx) push(k, k + 1, 1.0, 0.0, dy);
            else if (bcx == SWE_BC_PERIODIC) push(k, j * nx, 1.0, 0.0, dy);
            else push(k, -1, 1.0, 0.0, dy);
            if (j == 0 && bcy == SWE_BC_WALL) push(k, -1, 0.0, -1.0, dx);
            if (j + 1 < ny) push(k, k + nx, 0.0, 1.0, dx);
            else if (bcy == SWE_BC_PERIODIC) push(k, i, 0.0, 1.0, dx);
            else push(k, -1, 0.0, 1.0, dx);
        }
    if ((int64_t)out.a.size() >= (int64_t(1) << 30)) {
        err = "too many edges";
        return SWE_E_INVAL;
    }
    out.area.assign(N, dx * dy);
    finish_cells(N, out);
    return SWE_OK;
}

int build_tri_edges(int64_t nnodes, const double *xy, int64_t ncells, const int32_t *tri,
                    HostEdges &out, std::string &err)
{
    if (ncells < 1 || ncells > (int64_t(1) << 29)) {
        err = "ncells out of range";
        return SWE_E_INVAL;
    }
    out = HostEdges();
    out.area.resize(ncells);
    for (int64_t t = 0; t < ncells; ++t) {
        for (int k = 0; k < 3; ++k)
            if (tri[3 * t + k] < 0 || tri[3 * t + k] >= nnodes) {
                err = "node id out of range in triangle " + std::to_string(t);
                return SWE_E_INVAL;
            }
        const double *p0 = xy + 2 * (int64_t)tri[3 * t];
        const double *p1 = xy + 2 * (int64_t)tri[3 * t + 1];
        const double *p2 = xy + 2 * (int64_t)tri[3 * t + 2];
        const double ar = 0.5 * ((p1[0] - p0[0]) * (p2[1] - p0[1]) - (p2[0] - p0[0]) * (p1[1] - p0[1]));
        if (!(ar > 0.0)) {
            err = "triangle " + std::to_string(t) + " has non-positive area (not counter-clockwise?)";
            return SWE_E_INVAL;
        }
        out.area[t] = ar;
    }
    // pair up the 3 * ncells half-edges by their (min, max) node key
    struct Half {
        int64_t lo, hi;
        int32_t cell;
        int8_t k;
    };
    std::vector<Half> hs(3 * ncells);
    for (int64_t t = 0; t < ncells; ++t)
        for (int k = 0; k < 3; ++k) {
            const int64_t u = tri[3 * t + k], v = tri[3 * t + (k + 1) % 3];
            hs[3 * t + k] = Half{std::min(u, v), std::max(u, v), (int32_t)t, (int8_t)k};
        }
    std::sort(hs.begin(), hs.end(), [](const Half &x, const Half &y) {
        if (x.lo != y.lo) return x.lo < y.lo;
        if (x.hi != y.hi) return x.hi < y.hi;
        return x.cell < y.cell;
    });
    struct Ed {
        int32_t a, b;
        int8_t k;
    };
    std::vector<Ed> eds;
    eds.reserve(3 * ncells / 2 + 16);
    for (size_t i = 0; i < hs.size();) {
        size_t j = i + 1;
        while (j < hs.size() && hs[j].lo == hs[i].lo && hs[j].hi == hs[i].hi) ++j;
        if (j - i > 2) {
            err = "an edge is shared by more than two triangles";
            return SWE_E_INVAL;
        }
        if (j - i == 2) {
            if (hs[i].cell == hs[i + 1].cell) {
                err = "degenerate triangle repeats an edge";
                return SWE_E_INVAL;
            }
            eds.push_back(Ed{hs[i].cell, hs[i + 1].cell, hs[i].k}); // a = lower cell id
        } else {
            eds.push_back(Ed{hs[i].cell, -1, hs[i].k});
        }
        i = j;
    }
    // edges ordered by owner cell, then by the other cell
    std::sort(eds.begin(), eds.end(), [](const Ed &x, const Ed &y) {
        if (x.a != y.a) return x.a < y.a;
        return x.b < y.b;
    });
    const int64_t E = (int64_t)eds.size();
    out.a.resize(E);
    out.b.resize(E);
    out.nx.resize(E);
    out.ny.resize(E);
    out.len.resize(E);
    for (int64_t e = 0; e < E; ++e) {
        const int32_t t = eds[e].a;
        const int k = eds[e].k;
        const double *p = xy + 2 * (int64_t)tri[3 * t + k];
        const double *q = xy + 2 * (int64_t)tri[3 * t + (k + 1) % 3];
        const double ddx = q[0] - p[0], ddy = q[1] - p[1];
        const double len = std::sqrt(ddx * ddx + ddy * ddy);
        out.a[e] = t;
        out.b[e] = eds[e].b;
        out.nx[e] = ddy / len;
        out.ny[e] = -ddx / len;
        out.len[e] = len;
    }
    finish_cells(ncells, out);
    return SWE_OK;
}

// ---------------------------------------------------------------------------
// Morton order of triangle centroids
// ---------------------------------------------------------------------------

static uint64_t spread_bits16(uint64_t v)
{
    v &= 0xFFFFu;
    v = (v | (v << 8)) & 0x00FF00FFu;
    v = (v | (v << 4)) & 0x0F0F0F0Fu;
    v = (v | (v << 2)) & 0x33333333u;
    v = (v | (v << 1)) & 0x55555555u;
    return v;
}

void morton_perm(int64_t nnodes, const double *xy, int64_t ncells, const int32_t *tri,
                 std::vector<int32_t> &perm)
{
    (void)nnodes;
    std::vector<double> cx(ncells), cy(ncells);
    double x0 = 1e300, x1 = -1e300, y0 = 1e300, y1 = -1e300;
    for (int64_t t = 0; t < ncells; ++t) {
        double sx = 0, sy = 0;
        for (int k = 0; k < 3; ++k) {
            sx += xy[2 * (int64_t)tri[3 * t + k]];
            sy += xy[2 * (int64_t)tri[3 * t + k] + 1];
        }
        cx[t] = sx / 3.0;
        cy[t] = sy / 3.0;
        x0 = std::min(x0, cx[t]);
        x1 = std::max(x1, cx[t]);
        y0 = std::min(y0, cy[t]);
        y1 = std::max(y1, cy[t]);
    }
    const double sx = 65535.0 / std::max(x1 - x0, 1e-300), sy = 65535.0 / std::max(y1 - y0, 1e-300);
    std::vector<uint64_t> code(ncells);
    for (int64_t t = 0; t < ncells; ++t) {
        const uint64_t qx = (uint64_t)std::floor((cx[t] - x0) * sx);
        const uint64_t qy = (uint64_t)std::floor((cy[t] - y0) * sy);
        code[t] = spread_bits16(qx) | (spread_bits16(qy) << 1);
    }
    perm.resize(ncells);
    for (int64_t t = 0; t < ncells; ++t) perm[t] = (int32_t)t;
    std::stable_sort(perm.begin(), perm.end(), [&](int32_t a, int32_t b) { return code[a] < code[b]; });
}

// ---------------------------------------------------------------------------
// Blocks of the fused triangle path
// ---------------------------------------------------------------------------

// LDS banks (gfx950, measured): an 8-byte LDS read by a wavefront is served
// in two halves of 32 lanes, and a half takes as many cycles as the largest
// number of distinct addresses sharing one 8-byte bank slot, (address / 8)
// mod 32.  The kernels gather cell records of 7 reals by the cell's local id
// and fluctuation records of an odd number of reals by the record index, so
// two gathers share a slot exactly when their indices agree mod 32.  Two
// greedy passes spread them: the local edges are placed 32 at a time (the
// lanes of one half) so that the cells on each side of a half's edges differ
// mod 32 unless they are the same cell (one address, read once), and each
// updated cell's three slots are permuted within its half of cells so that
// each of the three gathers meets few shared slots.  Neither pass changes
// what is computed; the slot order only fixes the order of a cell's
// three-term sums.
struct BankSet {
    int32_t cell[32];
    void clear() { std::fill(cell, cell + 32, -1); }
    bool free_for(int32_t c) const { return c < 0 || cell[c & 31] < 0 || cell[c & 31] == c; }
    void put(int32_t c)
    {
        if (c >= 0 && cell[c & 31] < 0) cell[c & 31] = c;
    }
};

// Take n edges of rem into out for the current half (ua, ub: the cells on
// either side already in it): those that meet no shared slot, in order, then
// the leftovers that meet the fewest (among the first 64).
static void bank_take(std::vector<int32_t> &rem, int n, BankSet &ua, BankSet &ub, const std::vector<int32_t> &la,
                      const std::vector<int32_t> &lb, std::vector<int32_t> &out, std::vector<int32_t> &rest)
{
    rest.clear();
    int got = 0;
    for (int32_t k : rem) {
        if (got < n && ua.free_for(la[k]) && ub.free_for(lb[k])) {
            out.push_back(k);
            ua.put(la[k]);
            ub.put(lb[k]);
            ++got;
        } else {
            rest.push_back(k);
        }
    }
    while (got < n && !rest.empty()) {
        size_t best = 0;
        int bp = 3;
        for (size_t i = 0; i < rest.size() && i < 64; ++i) {
            const int p = !ua.free_for(la[rest[i]]) + !ub.free_for(lb[rest[i]]);
            if (p < bp) {
                bp = p;
                best = i;
            }
        }
        const int32_t k = rest[best];
        out.push_back(k);
        ua.put(la[k]);
        ub.put(lb[k]);
        rest.erase(rest.begin() + (ptrdiff_t)best);
        ++got;
    }
    rem.swap(rest);
}

// New order of a block's local edges (positions 0..ne-1 index la, lb: the
// local cells on either side, -1 for a wall); the first es0 stay first.
static void bank_order_edges(int es0, const std::vector<int32_t> &la, const std::vector<int32_t> &lb,
                             std::vector<int32_t> &order)
{
    const int ne = (int)la.size();
    std::vector<int32_t> ra, rb, rest;
    for (int k = 0; k < es0; ++k) ra.push_back(k);
    for (int k = es0; k < ne; ++k) rb.push_back(k);
    order.clear();
    BankSet ua, ub;
    while ((int)order.size() < ne) {
        ua.clear();
        ub.clear();
        int space = 32;
        const int na = std::min(space, (int)ra.size());
        bank_take(ra, na, ua, ub, la, lb, order, rest);
        space -= na;
        if (ra.empty() && space > 0) bank_take(rb, std::min(space, (int)rb.size()), ua, ub, la, lb, order, rest);
    }
}

// Permute each updated cell's three slots within its half of 32 cells.
static void bank_order_slots(HostBlocks &out)
{
    static const int P[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2}, {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
    std::vector<int32_t> used[3][32];
    for (int b = 0; b < out.nblocks; ++b) {
        const int s0 = out.slot_off[b], nc = out.slot_off[b + 1] - s0;
        for (int h0 = 0; h0 < nc; h0 += 32) {
            for (auto &u : used)
                for (auto &v : u) v.clear();
            for (int l = h0; l < std::min(nc, h0 + 32); ++l) {
                uint16_t *sl = &out.slots[4 * (size_t)(s0 + l)];
                int32_t r[3];
                for (int j = 0; j < 3; ++j) r[j] = (int32_t)((sl[j] & 1u) * (unsigned)out.e_max + (sl[j] >> 1));
                int best = 0, bp = 1 << 30;
                for (int q = 0; q < 6; ++q) {
                    int pen = 0;
                    for (int j = 0; j < 3; ++j) {
                        const std::vector<int32_t> &u = used[j][r[P[q][j]] & 31];
                        if (std::find(u.begin(), u.end(), r[P[q][j]]) == u.end()) pen += (int)u.size();
                    }
                    if (pen < bp) {
                        bp = pen;
                        best = q;
                    }
                }
                const uint16_t old[3] = {sl[0], sl[1], sl[2]};
                for (int j = 0; j < 3; ++j) {
                    sl[j] = old[P[best][j]];
                    std::vector<int32_t> &u = used[j][r[P[best][j]] & 31];
                    if (std::find(u.begin(), u.end(), r[P[best][j]]) == u.end()) u.push_back(r[P[best][j]]);
                }
            }
        }
    }
}

int build_tri_blocks(const HostEdges &he, int64_t N, int B, HostBlocks &out, std::string &err)
{
    out = HostBlocks();
    out.B = B;
    const int64_t E = (int64_t)he.a.size();
    const int nb = (int)((N + B - 1) / B);
    out.nblocks = nb;
    std::vector<int32_t> cstamp(N, -1), cloc(N, 0), estamp(E, -1), eloc(E, 0);
    out.halo_off.push_back(0);
    out.edge_off.push_back(0);
    out.slot_off.push_back(0);
    auto other = [&](int64_t e, int64_t c) -> int64_t { return he.a[e] == c ? he.b[e] : he.a[e]; };
    std::vector<int32_t> ring1, ring2, ledges;
    for (int b = 0; b < nb; ++b) {
        const int64_t base = (int64_t)b * B;
        const int B0 = (int)std::min<int64_t>(B, N - base);
        for (int l = 0; l < B0; ++l) {
            cstamp[base + l] = b;
            cloc[base + l] = l;
        }
        ring1.clear();
        ring2.clear();
        for (int l = 0; l < B0; ++l) {
            const int64_t c = base + l;
            for (int32_t k = he.off[c]; k < he.off[c + 1]; ++k) {
                const int64_t o = other(he.ce[k] >> 1, c);
                if (o >= 0 && cstamp[o] != b) {
                    cstamp[o] = b;
                    ring1.push_back((int32_t)o);
                }
            }
        }
        for (int32_t c : ring1)
            for (int32_t k = he.off[c]; k < he.off[c + 1]; ++k) {
                const int64_t o = other(he.ce[k] >> 1, c);
                if (o >= 0 && cstamp[o] != b) {
                    cstamp[o] = b;
                    ring2.push_back((int32_t)o);
                }
            }
        const int n1 = (int)ring1.size(), n2 = (int)ring2.size();
        for (int i = 0; i < n1; ++i) cloc[ring1[i]] = B0 + i;
        for (int i = 0; i < n2; ++i) cloc[ring2[i]] = B0 + n1 + i;
        const int lc = B0 + n1 + n2;
        // local edges: those of the block's cells first, then ring 1's
        ledges.clear();
        auto add_edges_of = [&](int64_t c) {
            for (int32_t k = he.off[c]; k < he.off[c + 1]; ++k) {
                const int32_t e = he.ce[k] >> 1;
                if (estamp[e] != b) {
                    estamp[e] = b;
                    eloc[e] = (int32_t)ledges.size();
                    ledges.push_back(e);
                }
            }
        };
        for (int l = 0; l < B0; ++l) add_edges_of(base + l);
        const int es0 = (int)ledges.size();
        for (int32_t c : ring1) add_edges_of(c);
        const int ne = (int)ledges.size();
        if (lc >= 0xFFFF || 2 * ne >= 0xFFFF) {
            err = "triangle block too large for 16-bit local indices";
            return SWE_E_INVAL;
        }
        {
            std::vector<int32_t> la(ne), lb(ne), order, tmp(ledges);
            for (int k = 0; k < ne; ++k) {
                la[k] = cloc[he.a[ledges[k]]];
                lb[k] = he.b[ledges[k]] >= 0 ? cloc[he.b[ledges[k]]] : -1;
            }
            bank_order_edges(es0, la, lb, order);
            for (int k = 0; k < ne; ++k) {
                ledges[k] = tmp[order[k]];
                eloc[ledges[k]] = k;
            }
        }
        for (int32_t e : ledges) {
            const uint32_t la = (uint32_t)cloc[he.a[e]];
            const uint32_t lb = he.b[e] >= 0 ? (uint32_t)cloc[he.b[e]] : 0xFFFFu;
            out.e_ab.push_back(la | (lb << 16));
            out.e_gx.push_back(he.len[e] * he.nx[e]);
            out.e_gy.push_back(he.len[e] * he.ny[e]);
        }
        auto add_slots_of = [&](int64_t c) {
            if (he.off[c + 1] - he.off[c] != 3) return false;
            for (int32_t k = he.off[c]; k < he.off[c + 1]; ++k) {
                const int32_t e = he.ce[k] >> 1, side = he.ce[k] & 1;
                out.slots.push_back((uint16_t)((eloc[e] << 1) | side));
            }
            out.slots.push_back(0); // padding: one 8-byte load per cell
            out.iarea.push_back(1.0 / he.area[c]);
            return true;
        };
        for (int l = 0; l < B0; ++l)
            if (!add_slots_of(base + l)) { err = "a triangle without three edges"; return SWE_E_INVAL; }
        for (int32_t c : ring1)
            if (!add_slots_of(c)) { err = "a triangle without three edges"; return SWE_E_INVAL; }
        out.halo_ids.insert(out.halo_ids.end(), ring1.begin(), ring1.end());
        out.halo_ids.insert(out.halo_ids.end(), ring2.begin(), ring2.end());
        out.halo_off.push_back((int32_t)out.halo_ids.size());
        out.n1.push_back(n1);
        out.e_s0.push_back(es0);
        out.edge_off.push_back((int32_t)out.e_ab.size());
        out.slot_off.push_back(out.slot_off.back() + B0 + n1);
        if (b == nb - 1) out.halo_ids.push_back(0); // padding: in-range clamped loads
        out.lc_max = std::max(out.lc_max, lc);
        out.e_max = std::max(out.e_max, ne);
    }
    bank_order_slots(out); // needs the final e_max (a record's index is side e_max + edge)
    return SWE_OK;
}

} // namespace swe
