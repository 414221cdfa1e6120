/* Test infrastructure: runs the oracle's time loops on inputs read from a
 * file, built with AddressSanitizer and UndefinedBehaviorSanitizer by the CPU
 * tests.  Only the oracle is linked.
 *
 * Input file (all int64 then doubles / int32):
 *   int64 kind (0 grid, 1 triangles, 2 two-layer triangles), int64 nsteps,
 *   int64 classical, int64 fix;
 *   grid:      int64 nx, ny, perx, pery; double dx, dy; double z[N], h, qx, qy, hc[N]
 *   triangles: int64 nnodes, ncells, ntracers; double xy[2 nnodes]; int32 tri[3 ncells];
 *              double z[N], h, qx, qy[N] (, hc[N])
 *   two-layer: int64 nnodes, ncells; double xy[]; int32 tri[]; double z, h1, q1x, q1y, h2, q2x, q2y
 * Prints the status and the sum of the dts. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int or_run_cart(int nx, int ny, double dx, double dy, int perx, int pery, double g, double cfl, int nsteps,
                const double *z, double *h, double *qx, double *qy, double *hc, double *dts, int nthreads,
                int classical, int fix);
int or_run_tri(int64_t nnodes, const double *xy, int64_t ncells, const int32_t *tri, double g, double cfl,
               int nsteps, const double *z, double *h, double *qx, double *qy, double *hc, double *dts, int nthreads,
               int classical, int fix);
int or_run_tri2(int64_t nnodes, const double *xy, int64_t ncells, const int32_t *tri, double g, double r, double cfl,
                int nsteps, const double *z, double *h1, double *q1x, double *q1y, double *h2, double *q2x,
                double *q2y, double *dts, int nthreads, int classical);

static FILE *f;
static void *owned[16];
static int nowned;
static void *keep(void *p)
{
    if (!p || nowned == 16) exit(2);
    return owned[nowned++] = p;
}
static int64_t rd64(void)
{
    int64_t v;
    if (fread(&v, 8, 1, f) != 1) exit(2);
    return v;
}
static double *rdd(int64_t n)
{
    double *p = keep(malloc((size_t)(n > 0 ? n : 1) * sizeof(double)));
    if (fread(p, 8, (size_t)n, f) != (size_t)n) exit(2);
    return p;
}
static int32_t *rdi(int64_t n)
{
    int32_t *p = keep(malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t)));
    if (fread(p, 4, (size_t)n, f) != (size_t)n) exit(2);
    return p;
}

int main(int argc, char **argv)
{
    if (argc != 2) return 2;
    f = fopen(argv[1], "rb");
    if (!f) return 2;
    const int64_t kind = rd64(), nsteps = rd64(), classical = rd64(), fix = rd64();
    double *dts = keep(malloc((size_t)(nsteps > 0 ? nsteps : 1) * sizeof(double)));
    int st;
    if (kind == 0) {
        const int64_t nx = rd64(), ny = rd64(), perx = rd64(), pery = rd64();
        double *d = rdd(2);
        const int64_t n = nx * ny;
        double *z = rdd(n), *h = rdd(n), *qx = rdd(n), *qy = rdd(n), *hc = rdd(n);
        st = or_run_cart((int)nx, (int)ny, d[0], d[1], (int)perx, (int)pery, 9.81, 0.9, (int)nsteps, z, h, qx, qy,
                         hc, dts, 2, (int)classical, (int)fix);
    } else if (kind == 1) {
        const int64_t nn = rd64(), nc = rd64(), ntr = rd64();
        double *xy = rdd(2 * nn);
        int32_t *tri = rdi(3 * nc);
        double *z = rdd(nc), *h = rdd(nc), *qx = rdd(nc), *qy = rdd(nc), *hc = ntr ? rdd(nc) : NULL;
        st = or_run_tri(nn, xy, nc, tri, 9.81, 0.9, (int)nsteps, z, h, qx, qy, hc, dts, 2, (int)classical, (int)fix);
    } else {
        const int64_t nn = rd64(), nc = rd64();
        double *xy = rdd(2 * nn);
        int32_t *tri = rdi(3 * nc);
        double *z = rdd(nc), *h1 = rdd(nc), *q1x = rdd(nc), *q1y = rdd(nc), *h2 = rdd(nc), *q2x = rdd(nc),
               *q2y = rdd(nc);
        st = or_run_tri2(nn, xy, nc, tri, 9.81, 0.98, 0.9, (int)nsteps, z, h1, q1x, q1y, h2, q2x, q2y, dts, 2,
                         (int)classical);
    }
    double t = 0.0;
    for (int64_t i = 0; i < nsteps; ++i) t += dts[i];
    printf("status %d t %.17g\n", st, t);
    fclose(f);
    for (int i = 0; i < nowned; ++i) free(owned[i]);
    return 0;
}
