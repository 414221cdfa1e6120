// Test infrastructure: runs the library's host-side mesh preprocessing (edge
// derivation, Morton order, per-block data of the fused triangle kernels,
// Cartesian edge lists) on meshes read from a file, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by the CPU tests, and checks the block data
// for internal consistency (local ids in range, every cell's three slots name
// edges of that cell on the right side, halo lists and offsets monotone).
//
// Input file: int64 nnodes, int64 ncells, double xy[2 nnodes], int32 tri[3 ncells].
// Exit status 0 and "ok" on success; 1 with a message on a failed check.
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../finite_volume_shallow_amd/csrc/swe_internal.hpp"

#define CHECK(cond, ...)                                                                    \
    do {                                                                                    \
        if (!(cond)) {                                                                      \
            std::printf("check failed: %s: ", #cond);                                       \
            std::printf(__VA_ARGS__);                                                       \
            std::printf("\n");                                                              \
            return 1;                                                                       \
        }                                                                                   \
    } while (0)

static int check_edges(const swe::HostEdges &he, int64_t ncells)
{
    const int64_t E = (int64_t)he.a.size();
    CHECK((int64_t)he.off.size() == ncells + 1, "offsets");
    for (int64_t c = 0; c < ncells; ++c) {
        CHECK(he.off[c] <= he.off[c + 1], "cell %lld", (long long)c);
        for (int32_t k = he.off[c]; k < he.off[c + 1]; ++k) {
            const int32_t e = he.ce[k] >> 1, side = he.ce[k] & 1;
            CHECK(e >= 0 && e < E, "edge id");
            CHECK((side ? he.b[e] : he.a[e]) == c, "cell %lld is not side %d of edge %d", (long long)c, side, e);
        }
    }
    for (int64_t e = 0; e < E; ++e) CHECK(he.len[e] > 0.0, "edge %lld length", (long long)e);
    return 0;
}

static int check_blocks(const swe::HostBlocks &hb, int64_t ncells)
{
    CHECK(hb.nblocks == (int)((ncells + hb.B - 1) / hb.B), "block count");
    for (int b = 0; b < hb.nblocks; ++b) {
        const int64_t base = (int64_t)b * hb.B;
        const int B0 = (int)std::min<int64_t>(hb.B, ncells - base);
        const int nh = hb.halo_off[b + 1] - hb.halo_off[b];
        const int lc = B0 + nh, n1 = hb.n1[b];
        CHECK(nh >= 0 && n1 >= 0 && n1 <= nh, "block %d halo", b);
        CHECK(lc <= hb.lc_max, "block %d local cells", b);
        for (int i = 0; i < nh; ++i) {
            const int32_t g = hb.halo_ids[hb.halo_off[b] + i];
            CHECK(g >= 0 && g < ncells && (g < base || g >= base + B0), "block %d halo id %d", b, g);
        }
        const int e0 = hb.edge_off[b], ne = hb.edge_off[b + 1] - e0;
        CHECK(ne >= 0 && ne <= hb.e_max && hb.e_s0[b] <= ne, "block %d edges", b);
        for (int k = 0; k < ne; ++k) {
            const uint32_t ab = hb.e_ab[e0 + k], la = ab & 0xFFFFu, lb = ab >> 16;
            CHECK((int)la < lc && (lb == 0xFFFFu || (int)lb < lc), "block %d edge %d cells %u %u", b, k, la, lb);
            // the edges touching the block come first (the kernels' speed phase takes those)
            const bool touches = (int)la < B0 || (lb != 0xFFFFu && (int)lb < B0);
            CHECK(touches == (k < hb.e_s0[b]), "block %d edge %d of %d touches the block: %d", b, k, hb.e_s0[b],
                  (int)touches);
        }
        const int s0 = hb.slot_off[b], nc = hb.slot_off[b + 1] - s0;
        CHECK(nc == B0 + n1, "block %d updated cells", b);
        for (int l = 0; l < nc; ++l) {
            CHECK(hb.iarea[s0 + l] > 0.0, "block %d cell %d area", b, l);
            for (int j = 0; j < 3; ++j) {
                const unsigned sl = hb.slots[4 * (size_t)(s0 + l) + j];
                const int k = (int)(sl >> 1), side = (int)(sl & 1);
                CHECK(k < ne, "block %d cell %d slot %d edge %d of %d", b, l, j, k, ne);
                const uint32_t ab = hb.e_ab[e0 + k];
                const uint32_t mine = side ? (ab >> 16) : (ab & 0xFFFFu);
                CHECK((int)mine == l, "block %d cell %d slot %d names cell %u", b, l, j, mine);
            }
            const uint16_t *sl = &hb.slots[4 * (size_t)(s0 + l)];
            CHECK(sl[0] != sl[1] && sl[0] != sl[2] && sl[1] != sl[2], "block %d cell %d repeats a slot", b, l);
        }
    }
    return 0;
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        std::printf("usage: mesh_harness MESHFILE\n");
        return 2;
    }
    FILE *f = std::fopen(argv[1], "rb");
    if (!f) return 2;
    int64_t nn = 0, nc = 0;
    if (std::fread(&nn, 8, 1, f) != 1 || std::fread(&nc, 8, 1, f) != 1) return 2;
    std::vector<double> xy((size_t)(2 * nn));
    std::vector<int32_t> tri((size_t)(3 * nc));
    if (std::fread(xy.data(), 8, xy.size(), f) != xy.size() || std::fread(tri.data(), 4, tri.size(), f) != tri.size())
        return 2;
    std::fclose(f);

    std::string err;
    swe::HostEdges he;
    if (swe::build_tri_edges(nn, xy.data(), nc, tri.data(), he, err) != SWE_OK) {
        std::printf("rejected: %s\n", err.c_str());
        return 3;
    }
    if (check_edges(he, nc)) return 1;

    // internal (Morton) order, as the fused path builds it
    std::vector<int32_t> perm;
    swe::morton_perm(nn, xy.data(), nc, tri.data(), perm);
    CHECK((int64_t)perm.size() == nc, "permutation size");
    std::vector<char> seen((size_t)nc, 0);
    for (int32_t p : perm) {
        CHECK(p >= 0 && p < nc && !seen[p], "permutation entry %d", p);
        seen[p] = 1;
    }
    std::vector<int32_t> tri_int((size_t)(3 * nc));
    for (int64_t i = 0; i < nc; ++i)
        for (int k = 0; k < 3; ++k) tri_int[3 * i + k] = tri[3 * (int64_t)perm[i] + k];
    swe::HostEdges hi;
    if (swe::build_tri_edges(nn, xy.data(), nc, tri_int.data(), hi, err) != SWE_OK) {
        std::printf("internal order rejected: %s\n", err.c_str());
        return 1;
    }
    if (check_edges(hi, nc)) return 1;
    for (int B : {32, 64, 96, 128, 192, 224, 288, 512}) {
        swe::HostBlocks hb;
        if (swe::build_tri_blocks(hi, nc, B, hb, err) != SWE_OK) {
            std::printf("blocks of %d: %s\n", B, err.c_str());
            continue;
        }
        if (check_blocks(hb, nc)) return 1;
    }

    // Cartesian edge lists of a few small grids, walls and periodic sides
    for (int64_t nx : {2, 3, 7})
        for (int64_t ny : {2, 5})
            for (int bx = 0; bx < 2; ++bx)
                for (int by = 0; by < 2; ++by) {
                    swe::HostEdges hc;
                    if (swe::build_cart_edges(nx, ny, 1.0, 2.0, bx, by, hc, err) != SWE_OK) {
                        std::printf("grid %lldx%lld: %s\n", (long long)nx, (long long)ny, err.c_str());
                        return 1;
                    }
                    if (check_edges(hc, nx * ny)) return 1;
                }
    std::printf("ok\n");
    return 0;
}
