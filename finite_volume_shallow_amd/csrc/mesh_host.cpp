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

} // namespace swe
