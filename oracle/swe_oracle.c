/*
 * Plain fp64 CPU oracle for one explicit step of the first-order Roe
 * finite-volume scheme for the 2D shallow-water equations.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the GPU library against an
 * obviously correct, slow implementation that shares no code with it.
 *
 * Sources (the pages this follows):
 *  [IR] de la Asuncion, Mantas, Castro, Fernandez-Nieto, "An MPI-CUDA
 *       implementation of an improved Roe method for two-layer shallow water
 *       systems": Sec. 2.1 Eq. (1) (model, matrices B_k, S_k, P_{l,k}),
 *       Eqs. (2)-(3) (rotation T_eta), Sec. 2.2 Eq. (4) (finite-volume
 *       update), steps 1-4 of the IR-Roe flux (Roe matrix A_ij, averages,
 *       P^- = 1/2 K (I - sgn D) K^-1, the upwinded transverse flux) and
 *       Eq. (5) (CFL condition).
 *  [MG] Vinas et al., "A multi-GPU shallow-water simulation with transport
 *       of contaminants": abstract (one-layer SWE + a transport equation for
 *       the pollutant, first-order Roe finite volumes).
 *
 * Readings where the pages are silent or garbled (each is listed in the
 * design notes of the repository as well):
 *  - The density ratio r lost in extraction sits in the lower-layer coupling:
 *    the lower-layer momentum equation carries -r g h2 d(h1); row 4 of A_ij
 *    is (r g h2, 0, g h2 - u2^2, 2 u2).  The upper layer carries no r.
 *  - Eq. (4) reads W_i^{n+1} = W_i^n - dt/|V_i| sum_j |G_ij| F^-_ij.
 *  - H = -z (depth below a fixed reference); only H_j - H_i enters.
 *  - B_ij and S_ij are evaluated with the arithmetic-mean depths of the
 *    Roe state (the pages define h_k,ij exactly there).
 *  - sgn(0) = 0, so a wave of zero speed is split half and half.
 *  - The upwind choice for the transverse momentum and the pollutant takes
 *    the left state when the mass flux is > 0, else the right state.
 *  - No entropy fix by default.  [IR] Sec. 2.2 only says the Harten-Hyman
 *    fix of its ref. [25] can be adapted; the optional one here (one layer,
 *    IR-Roe or classical) is that fix in its wave-splitting form, applied to the
 *    conservative part of each acoustic wave: with b = K^-1 (W_R - W_L) the
 *    state jumps of the Roe waves and W* = W_L + b_1 r_1 the state between
 *    them, a wave k whose characteristic speed is < 0 on its left state and
 *    > 0 on its right state (a transonic rarefaction) is split into a part
 *    of speed lam_left going left and one of speed lam_right going right,
 *    with the fraction (lam_right - lam_k)/(lam_right - lam_left) going left,
 *    so that its left-going flux jump min(lam_k, 0) b_k r_k becomes
 *    lam_left (lam_right - lam_k)/(lam_right - lam_left) b_k r_k.  The
 *    source part of the wave is untouched (a lake at rest has no transonic
 *    wave, so the fix keeps the scheme well-balanced).
 *  - The pollutant is a passive scalar carried by the mass flux, upwinded
 *    like the transverse momentum of step 3 ([MG] gives no other flux).
 *  - Reflective wall = mirror ghost (normal momentum negated) pushed through
 *    the same Roe flux; its mass, transverse and pollutant fluxes are set to
 *    exactly zero.  For one layer the remaining momentum flux is the closed
 *    form q^2/h + g h^2/2 + sqrt(g h) q of that mirror problem.
 *  - Periodic sides wrap to the opposite cell.
 *  - The time step is taken from the state at the start of the step (the
 *    wave speeds come from the same edge pass as the fluxes), dt = min_i of
 *    2 gamma |V_i| / sum_j |G_ij| ||D_ij||_inf over all cells.
 *
 * Classical Roe variant (one layer, selected per run): the full Roe matrix
 * of the edge-normal system in (h, q_n, q_t, hc) -- its transverse momentum
 * and pollutant rows carry contact waves of speed u_Roe -- upwinded with
 * P^- = K (1/2 (I - sgn D)) K^-1 on all four waves, in place of the IR-Roe
 * step 3 (transverse momentum and pollutant upwinded by the sign of the mass
 * flux).  The pages contrast the two schemes; the classical one is the
 * reference the IR-Roe method improves on.  Same walls and same Eq. (5).
 * Two layers: the full 6x6 Roe matrix of (h1, q1n, q1t, h2, q2n, q2t) --
 * the 4x4 matrix A_ij of the normal system plus the transverse rows of each
 * layer, linearised at that layer's Roe averages -- eigen-decomposed as a
 * whole (K of 6 columns, K alpha = X solved by elimination).
 *
 * The flux is evaluated per cell from that cell's own side, literally as in
 * Eq. (4): every interior edge is therefore computed twice, once from each
 * side, with the outward normal of the cell being updated.
 *
 * Parity pins: see the oracle tests.  The two-layer eigen-solver (Faddeev-
 * LeVerrier characteristic polynomial + Durand-Kerner roots + adjugate
 * eigenvectors + Gaussian elimination) is pinned against a generic library
 * eigen-decomposition and the closed form at equal layer velocities.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    OR_OK = 0,
    OR_BADMESH = 1,
    OR_DEPTH = 2,
    OR_NONFINITE = 3,
    OR_NONHYPERBOLIC = 4,
    OR_NOMEM = 5,
    OR_NOCONV = 6
};

static double sgn(double x) { return (x > 0.0) - (x < 0.0); }

/* ------------------------------------------------------------------------ */
/* One layer: 1D Roe flux in the frame of the edge normal ([IR] Sec. 2.2,   */
/* steps 1-3 with a single layer; 2x2 Roe matrix A = [[0,1],[g h - u^2,2u]]) */
/* ------------------------------------------------------------------------ */

/* L, R: (h, q_normal, q_transverse, hc, H).  phi: (mass, normal momentum,
 * transverse momentum, pollutant) flux leaving L through the edge.  speed:
 * max |eigenvalue| of the Roe matrix. */
/* Harten-Hyman correction of the left-going flux jump (P0, P1) of the
 * one-layer 2x2 Roe solution (see the header): lam1, lam2 the Roe speeds. */
static void hh_fix(const double *L, const double *R, double g, double lam1,
                   double lam2, double *P0, double *P1)
{
    double hL = L[0], qL = L[1], hR = R[0], qR = R[1];
    double dh = hR - hL, dq = qR - qL;
    double b1 = (lam2 * dh - dq) / (lam2 - lam1);  /* K^-1 (W_R - W_L) */
    double b2 = (dq - lam1 * dh) / (lam2 - lam1);
    double hs = hL + b1, qs = qL + b1 * lam1;       /* W* */
    if (!(hs > 0.0)) return;
    double us = qs / hs, cs = sqrt(g * hs);
    double uL = qL / hL, uR = qR / hR;
    /* wave 1 between W_L and W*, wave 2 between W* and W_R */
    double l1L = uL - sqrt(g * hL), l1R = us - cs;
    double l2L = us + cs, l2R = uR + sqrt(g * hR);
    if (l1L < 0.0 && l1R > 0.0) {
        double lb = l1L * (l1R - lam1) / (l1R - l1L);
        double corr = lb - fmin(lam1, 0.0);
        *P0 += corr * b1;
        *P1 += corr * b1 * lam1;
    }
    if (l2L < 0.0 && l2R > 0.0) {
        double lb = l2L * (l2R - lam2) / (l2R - l2L);
        double corr = lb - fmin(lam2, 0.0);
        *P0 += corr * b2;
        *P1 += corr * b2 * lam2;
    }
}

static int roe1_ir(const double *L, const double *R, double g, int fix,
                   double *phi, double *speed);

int or_roe1_edge(const double *L, const double *R, double g, double *phi,
                 double *speed)
{
    return roe1_ir(L, R, g, 0, phi, speed);
}

/* As or_roe1_edge, with the Harten-Hyman entropy fix when fix != 0. */
int or_roe1_edge_fix(const double *L, const double *R, double g, int fix,
                     double *phi, double *speed)
{
    return roe1_ir(L, R, g, fix, phi, speed);
}

static int roe1_ir(const double *L, const double *R, double g, int fix,
                   double *phi, double *speed)
{
    double hL = L[0], qL = L[1], tL = L[2], cL = L[3], HL = L[4];
    double hR = R[0], qR = R[1], tR = R[2], cR = R[3], HR = R[4];
    if (!(hL > 0.0) || !(hR > 0.0)) return OR_DEPTH;

    double uL = qL / hL, uR = qR / hR;
    double sL = sqrt(hL), sR = sqrt(hR);
    double ubar = (sL * uL + sR * uR) / (sL + sR);   /* Roe velocity     */
    double hbar = 0.5 * (hL + hR);                     /* arithmetic mean  */
    double c = sqrt(g * hbar);
    double lam1 = ubar - c, lam2 = ubar + c;           /* eigenvalues of A */

    /* F1 of the 1D system and the path-conservative difference
     * X = F(W_R) - F(W_L) - S (H_R - H_L), S = (0, g hbar). */
    double FL0 = qL, FL1 = qL * qL / hL + 0.5 * g * hL * hL;
    double FR0 = qR, FR1 = qR * qR / hR + 0.5 * g * hR * hR;
    double X0 = FR0 - FL0;
    double X1 = FR1 - FL1 - g * hbar * (HR - HL);

    /* K = [[1, 1], [lam1, lam2]]; alpha = K^-1 X. */
    double a1 = (lam2 * X0 - X1) / (lam2 - lam1);
    double a2 = (X1 - lam1 * X0) / (lam2 - lam1);
    double w1 = 0.5 * (1.0 - sgn(lam1));
    double w2 = 0.5 * (1.0 - sgn(lam2));
    double P0 = w1 * a1 + w2 * a2;
    double P1 = w1 * a1 * lam1 + w2 * a2 * lam2;
    if (fix) hh_fix(L, R, g, lam1, lam2, &P0, &P1);

    double f0 = FL0 + P0;
    double f1 = FL1 + P1;
    /* step 3: passive scalars carried by the mass flux, upwinded */
    double ustar = (f0 > 0.0) ? tL / hL : tR / hR;
    double cstar = (f0 > 0.0) ? cL / hL : cR / hR;
    phi[0] = f0;
    phi[1] = f1;
    phi[2] = f0 * ustar;
    phi[3] = f0 * cstar;
    *speed = fmax(fabs(lam1), fabs(lam2));
    return OR_OK;
}

/* Classical Roe flux for the same edge states.  Roe matrix of the system
 * (h, q_n, q_t, hc) with flux (q_n, q_n^2/h + g h^2/2, q_n q_t/h, q_n hc/h)
 * at the Roe state (u, v, C Roe averages of the normal and transverse
 * velocities and the concentration, c^2 = g hbar):
 *   A = [[0, 1, 0, 0], [c^2 - u^2, 2u, 0, 0], [-u v, v, u, 0], [-u C, C, 0, u]]
 * eigenvalues u - c, u, u, u + c with right eigenvectors
 *   r1 = (1, u - c, v, C), r2 = (0, 0, 1, 0), r3 = (0, 0, 0, 1), r4 = (1, u + c, v, C).
 * X = F(W_R) - F(W_L) - S (H_R - H_L); alpha = K^-1 X; Phi = F(W_L) + P^- X. */
static int roe1_classical(const double *L, const double *R, double g, int fix,
                          double *phi, double *speed);

int or_roe1c_edge(const double *L, const double *R, double g, double *phi,
                  double *speed)
{
    return roe1_classical(L, R, g, 0, phi, speed);
}

/* As or_roe1c_edge, with the Harten-Hyman entropy fix on its two acoustic
 * waves when fix != 0 (the contact waves are linearly degenerate: no fix). */
int or_roe1c_edge_fix(const double *L, const double *R, double g, int fix,
                      double *phi, double *speed)
{
    return roe1_classical(L, R, g, fix, phi, speed);
}

static int roe1_classical(const double *L, const double *R, double g, int fix,
                          double *phi, double *speed)
{
    double hL = L[0], qL = L[1], tL = L[2], cL = L[3], HL = L[4];
    double hR = R[0], qR = R[1], tR = R[2], cR = R[3], HR = R[4];
    if (!(hL > 0.0) || !(hR > 0.0)) return OR_DEPTH;

    double uL = qL / hL, uR = qR / hR, vL = tL / hL, vR = tR / hR;
    double kL = cL / hL, kR = cR / hR; /* concentrations */
    double sL = sqrt(hL), sR = sqrt(hR);
    double ubar = (sL * uL + sR * uR) / (sL + sR);
    double vbar = (sL * vL + sR * vR) / (sL + sR);
    double Cbar = (sL * kL + sR * kR) / (sL + sR);
    double hbar = 0.5 * (hL + hR);
    double c = sqrt(g * hbar);
    double lam[4] = {ubar - c, ubar, ubar, ubar + c};

    double FL[4] = {qL, qL * qL / hL + 0.5 * g * hL * hL, qL * vL, qL * kL};
    double FR[4] = {qR, qR * qR / hR + 0.5 * g * hR * hR, qR * vR, qR * kR};
    double X[4];
    for (int v = 0; v < 4; ++v) X[v] = FR[v] - FL[v];
    X[1] -= g * hbar * (HR - HL);

    /* alpha = K^-1 X for K = [r1 r2 r3 r4] */
    double al[4];
    al[0] = (lam[3] * X[0] - X[1]) / (lam[3] - lam[0]);
    al[3] = (X[1] - lam[0] * X[0]) / (lam[3] - lam[0]);
    al[1] = X[2] - vbar * X[0]; /* rows 3, 4 of K alpha = X: alpha1 + alpha4 = X0 */
    al[2] = X[3] - Cbar * X[0];
    double r[4][4] = {{1.0, lam[0], vbar, Cbar},
                      {0.0, 0.0, 1.0, 0.0},
                      {0.0, 0.0, 0.0, 1.0},
                      {1.0, lam[3], vbar, Cbar}};
    for (int v = 0; v < 4; ++v) phi[v] = FL[v];
    for (int k = 0; k < 4; ++k) {
        double w = 0.5 * (1.0 - sgn(lam[k]));
        for (int v = 0; v < 4; ++v) phi[v] += w * al[k] * r[k][v];
    }
    if (fix) { /* the fix's change of the acoustic waves, along r1 and r4 */
        double d0 = 0.0, d1 = 0.0;
        hh_fix(L, R, g, lam[0], lam[3], &d0, &d1);
        phi[0] += d0;
        phi[1] += d1;
        phi[2] += vbar * d0;
        phi[3] += Cbar * d0;
    }
    *speed = fmax(fabs(lam[0]), fabs(lam[3]));
    return OR_OK;
}

/* Reflective wall: the mirror ghost problem in closed form. */
int or_roe1_wall(const double *L, double g, double *phi, double *speed)
{
    double h = L[0], q = L[1];
    if (!(h > 0.0)) return OR_DEPTH;
    double c = sqrt(g * h);
    phi[0] = 0.0;
    phi[1] = q * q / h + 0.5 * g * h * h + c * q;
    phi[2] = 0.0;
    phi[3] = 0.0;
    *speed = c;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Two layers ([IR] Sec. 2.2 steps 1-4, 4x4 Roe matrix A_ij)                */
/* ------------------------------------------------------------------------ */

static double det3(double a, double b, double c, double d, double e, double f,
                   double g, double h, double i)
{
    return a * (e * i - f * h) - b * (d * i - f * g) + c * (d * h - e * g);
}

/* Characteristic polynomial det(x I - A) = x^4 + p[3] x^3 + ... + p[0]
 * by the Faddeev-LeVerrier recursion. */
static void charpoly4(const double A[4][4], double p[5])
{
    double M[4][4] = {{0}}, AM[4][4];
    double c = 1.0;
    p[4] = 1.0;
    for (int k = 1; k <= 4; ++k) {
        /* M_k = A M_{k-1} + c_{n-k+1} I */
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j) {
                double s = 0.0;
                for (int l = 0; l < 4; ++l) s += A[i][l] * M[l][j];
                AM[i][j] = s;
            }
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j) M[i][j] = AM[i][j] + (i == j ? c : 0.0);
        double tr = 0.0;
        for (int i = 0; i < 4; ++i)
            for (int l = 0; l < 4; ++l) tr += A[i][l] * M[l][i];
        c = -tr / k;
        p[4 - k] = c;
    }
}

static double complex peval(const double p[5], double complex x)
{
    double complex s = p[4];
    for (int k = 3; k >= 0; --k) s = s * x + p[k];
    return s;
}

/* Durand-Kerner (Weierstrass) iteration for the four roots of a monic
 * quartic, then Newton polishing of the real parts. */
static int quartic_roots(const double p[5], double lam[4])
{
    double bound = 1.0;
    for (int k = 0; k < 4; ++k) bound = fmax(bound, 1.0 + fabs(p[k]));
    double complex z[4];
    for (int k = 0; k < 4; ++k)
        z[k] = 0.5 * bound * cexp(I * (0.4 + 2.0 * M_PI * k / 4.0));
    int converged = 0, extra = 0;
    for (int it = 0; it < 5000; ++it) {
        double maxd = 0.0, maxz = 0.0;
        for (int k = 0; k < 4; ++k) {
            double complex den = 1.0;
            for (int j = 0; j < 4; ++j)
                if (j != k) den *= (z[k] - z[j]);
            double complex d = peval(p, z[k]) / den;
            z[k] -= d;
            maxd = fmax(maxd, cabs(d));
            maxz = fmax(maxz, cabs(z[k]));
        }
        if (maxd <= 1e-15 * (1.0 + maxz)) {
            if (++extra >= 3) { converged = 1; break; }
        }
    }
    if (!converged) return OR_NOCONV;
    double maxabs = 0.0;
    for (int k = 0; k < 4; ++k) maxabs = fmax(maxabs, cabs(z[k]));
    for (int k = 0; k < 4; ++k)
        if (fabs(cimag(z[k])) > 1e-8 * maxabs) return OR_NONHYPERBOLIC;
    for (int k = 0; k < 4; ++k) {
        double x = creal(z[k]);
        for (int it = 0; it < 3; ++it) {
            double f = p[4], df = 0.0;
            for (int j = 3; j >= 0; --j) { df = df * x + f; f = f * x + p[j]; }
            if (df != 0.0) x -= f / df;
        }
        lam[k] = x;
    }
    /* ascending order (insertion sort) */
    for (int i = 1; i < 4; ++i) {
        double v = lam[i];
        int j = i - 1;
        while (j >= 0 && lam[j] > v) { lam[j + 1] = lam[j]; --j; }
        lam[j + 1] = v;
    }
    return OR_OK;
}

/* A null vector of the (numerically) singular M = A - lam I: the row of
 * cofactors with the largest norm (a column of adj(M)). */
static void null_vector4(const double M[4][4], double v[4])
{
    double best = -1.0;
    for (int r = 0; r < 4; ++r) {
        int rows[3], n = 0;
        for (int i = 0; i < 4; ++i)
            if (i != r) rows[n++] = i;
        double cof[4], nrm = 0.0;
        for (int c = 0; c < 4; ++c) {
            int cols[3], m = 0;
            for (int j = 0; j < 4; ++j)
                if (j != c) cols[m++] = j;
            double d = det3(M[rows[0]][cols[0]], M[rows[0]][cols[1]], M[rows[0]][cols[2]],
                            M[rows[1]][cols[0]], M[rows[1]][cols[1]], M[rows[1]][cols[2]],
                            M[rows[2]][cols[0]], M[rows[2]][cols[1]], M[rows[2]][cols[2]]);
            cof[c] = ((r + c) % 2 ? -d : d);
            nrm += cof[c] * cof[c];
        }
        if (nrm > best) {
            best = nrm;
            double s = 1.0 / sqrt(nrm);
            for (int c = 0; c < 4; ++c) v[c] = cof[c] * s;
        }
    }
}

/* Solve K a = x by Gaussian elimination with partial pivoting. */
static int solve4(const double Kin[4][4], const double x[4], double a[4])
{
    double K[4][5];
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j) K[i][j] = Kin[i][j];
        K[i][4] = x[i];
    }
    for (int c = 0; c < 4; ++c) {
        int piv = c;
        for (int i = c + 1; i < 4; ++i)
            if (fabs(K[i][c]) > fabs(K[piv][c])) piv = i;
        if (K[piv][c] == 0.0) return OR_NONHYPERBOLIC;
        if (piv != c)
            for (int j = 0; j < 5; ++j) {
                double t = K[c][j]; K[c][j] = K[piv][j]; K[piv][j] = t;
            }
        for (int i = c + 1; i < 4; ++i) {
            double f = K[i][c] / K[c][c];
            for (int j = c; j < 5; ++j) K[i][j] -= f * K[c][j];
        }
    }
    for (int i = 3; i >= 0; --i) {
        double s = K[i][4];
        for (int j = i + 1; j < 4; ++j) s -= K[i][j] * a[j];
        a[i] = s / K[i][i];
    }
    return OR_OK;
}

/* L, R: (h1, q1_normal, q1_transverse, h2, q2_normal, q2_transverse, H).
 * phi: the six components of F^- in the edge frame, ordered as W:
 * (h1, q1n, q1t, h2, q2n, q2t).  lam: the four eigenvalues, ascending. */
int or_roe2_edge(const double *L, const double *R, double g, double r,
                 double *phi, double *speed, double *lam)
{
    double h1L = L[0], q1L = L[1], t1L = L[2], h2L = L[3], q2L = L[4], t2L = L[5], HL = L[6];
    double h1R = R[0], q1R = R[1], t1R = R[2], h2R = R[3], q2R = R[4], t2R = R[5], HR = R[6];
    if (!(h1L > 0.0) || !(h2L > 0.0) || !(h1R > 0.0) || !(h2R > 0.0)) return OR_DEPTH;

    /* Roe averages per layer */
    double s1L = sqrt(h1L), s1R = sqrt(h1R), s2L = sqrt(h2L), s2R = sqrt(h2R);
    double u1 = (s1L * (q1L / h1L) + s1R * (q1R / h1R)) / (s1L + s1R);
    double u2 = (s2L * (q2L / h2L) + s2R * (q2R / h2R)) / (s2L + s2R);
    double h1 = 0.5 * (h1L + h1R), h2 = 0.5 * (h2L + h2R);

    /* A_ij = J_ij - B_ij on the reduced unknowns (h1, q1, h2, q2). */
    double J[4][4] = {{0.0, 1.0, 0.0, 0.0},
                      {g * h1 - u1 * u1, 2.0 * u1, 0.0, 0.0},
                      {0.0, 0.0, 0.0, 1.0},
                      {0.0, 0.0, g * h2 - u2 * u2, 2.0 * u2}};
    double B[4][4] = {{0.0, 0.0, 0.0, 0.0},
                      {0.0, 0.0, -g * h1, 0.0},
                      {0.0, 0.0, 0.0, 0.0},
                      {-r * g * h2, 0.0, 0.0, 0.0}};
    double S[4] = {0.0, g * h1, 0.0, g * h2};
    double A[4][4];
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) A[i][j] = J[i][j] - B[i][j];

    double p[5], ev[4];
    charpoly4(A, p);
    int st = quartic_roots(p, ev);
    if (st != OR_OK) return st;

    double K[4][4];
    for (int k = 0; k < 4; ++k) {
        double M[4][4], v[4];
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j) M[i][j] = A[i][j] - (i == j ? ev[k] : 0.0);
        null_vector4(M, v);
        for (int i = 0; i < 4; ++i) K[i][k] = v[i];
    }

    double FL[4] = {q1L, q1L * q1L / h1L + 0.5 * g * h1L * h1L,
                    q2L, q2L * q2L / h2L + 0.5 * g * h2L * h2L};
    double FR[4] = {q1R, q1R * q1R / h1R + 0.5 * g * h1R * h1R,
                    q2R, q2R * q2R / h2R + 0.5 * g * h2R * h2R};
    double dW[4] = {h1R - h1L, q1R - q1L, h2R - h2L, q2R - q2L};
    double X[4];
    for (int i = 0; i < 4; ++i) {
        double BdW = 0.0;
        for (int j = 0; j < 4; ++j) BdW += B[i][j] * dW[j];
        X[i] = FR[i] - FL[i] - BdW - S[i] * (HR - HL);
    }
    double alpha[4];
    st = solve4(K, X, alpha);
    if (st != OR_OK) return st;

    double PX[4] = {0.0, 0.0, 0.0, 0.0};
    for (int k = 0; k < 4; ++k) {
        double w = 0.5 * (1.0 - sgn(ev[k]));
        for (int i = 0; i < 4; ++i) PX[i] += w * alpha[k] * K[i][k];
    }
    double f[4];
    for (int i = 0; i < 4; ++i) f[i] = FL[i] + PX[i];

    double u1s = (f[0] > 0.0) ? t1L / h1L : t1R / h1R;
    double u2s = (f[2] > 0.0) ? t2L / h2L : t2R / h2R;
    phi[0] = f[0];
    phi[1] = f[1];
    phi[2] = f[0] * u1s;
    phi[3] = f[2];
    phi[4] = f[3];
    phi[5] = f[2] * u2s;
    double m = 0.0;
    for (int k = 0; k < 4; ++k) m = fmax(m, fabs(ev[k]));
    *speed = m;
    if (lam)
        for (int k = 0; k < 4; ++k) lam[k] = ev[k];
    return OR_OK;
}

/* Solve K a = x (n <= 6) by Gaussian elimination with partial pivoting. */
static int solve_n(int n, const double Kin[6][6], const double x[6], double a[6])
{
    double K[6][7];
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < n; ++j) K[i][j] = Kin[i][j];
        K[i][n] = x[i];
    }
    for (int c = 0; c < n; ++c) {
        int piv = c;
        for (int i = c + 1; i < n; ++i)
            if (fabs(K[i][c]) > fabs(K[piv][c])) piv = i;
        if (K[piv][c] == 0.0) return OR_NONHYPERBOLIC;
        if (piv != c)
            for (int j = 0; j <= n; ++j) {
                double t = K[c][j]; K[c][j] = K[piv][j]; K[piv][j] = t;
            }
        for (int i = c + 1; i < n; ++i) {
            double f = K[i][c] / K[c][c];
            for (int j = c; j <= n; ++j) K[i][j] -= f * K[c][j];
        }
    }
    for (int i = n - 1; i >= 0; --i) {
        double s = K[i][n];
        for (int j = i + 1; j < n; ++j) s -= K[i][j] * a[j];
        a[i] = s / K[i][i];
    }
    return OR_OK;
}

/* Classical Roe flux, two layers: P^- X with the full 6x6 Roe matrix of the
 * edge-normal system in W6 = (h1, q1n, q1t, h2, q2n, q2t).  Rows h_k and
 * q_kn are those of A_ij (J_ij - B_ij); the row of q_kt is the Roe
 * linearisation of its flux q_kn q_kt / h_k, (-u_k v_k, v_k, u_k) on
 * (h_k, q_kn, q_kt), with v_k the sqrt(h)-weighted average of q_kt / h_k.
 * The matrix is block triangular (the normal unknowns do not see q_kt), so
 * its eigenvalues are the four of A_ij and u1, u2; the eigenvectors of
 * u1, u2 are the unit vectors of q1t, q2t, and those of A_ij's eigenvalues
 * are A_ij's eigenvectors completed by the q_kt rows of (A6 - lam I) v = 0.
 * The transverse rows of X carry no bed or coupling term.
 * L, R, phi, speed, lam: as or_roe2_edge (lam: A_ij's four eigenvalues). */
int or_roe2c_edge(const double *L, const double *R, double g, double r,
                  double *phi, double *speed, double *lam)
{
    double h1L = L[0], q1L = L[1], t1L = L[2], h2L = L[3], q2L = L[4], t2L = L[5], HL = L[6];
    double h1R = R[0], q1R = R[1], t1R = R[2], h2R = R[3], q2R = R[4], t2R = R[5], HR = R[6];
    if (!(h1L > 0.0) || !(h2L > 0.0) || !(h1R > 0.0) || !(h2R > 0.0)) return OR_DEPTH;

    double s1L = sqrt(h1L), s1R = sqrt(h1R), s2L = sqrt(h2L), s2R = sqrt(h2R);
    double u1 = (s1L * (q1L / h1L) + s1R * (q1R / h1R)) / (s1L + s1R);
    double u2 = (s2L * (q2L / h2L) + s2R * (q2R / h2R)) / (s2L + s2R);
    double v1 = (s1L * (t1L / h1L) + s1R * (t1R / h1R)) / (s1L + s1R);
    double v2 = (s2L * (t2L / h2L) + s2R * (t2R / h2R)) / (s2L + s2R);
    double h1 = 0.5 * (h1L + h1R), h2 = 0.5 * (h2L + h2R);

    /* A6 = J6 - B6; B6 and the source S6 act on the normal rows only */
    double A[6][6] = {{0.0, 1.0, 0.0, 0.0, 0.0, 0.0},
                      {g * h1 - u1 * u1, 2.0 * u1, 0.0, g * h1, 0.0, 0.0},
                      {-u1 * v1, v1, u1, 0.0, 0.0, 0.0},
                      {0.0, 0.0, 0.0, 0.0, 1.0, 0.0},
                      {r * g * h2, 0.0, 0.0, g * h2 - u2 * u2, 2.0 * u2, 0.0},
                      {0.0, 0.0, 0.0, -u2 * v2, v2, u2}};
    double B[6][6] = {{0.0}};
    B[1][3] = -g * h1;
    B[4][0] = -r * g * h2;
    double S[6] = {0.0, g * h1, 0.0, 0.0, g * h2, 0.0};

    /* eigenvalues: those of the normal block (rows/columns h1, q1n, h2, q2n) */
    static const int nb[4] = {0, 1, 3, 4};
    double A4[4][4], p[5], ev[4];
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) A4[i][j] = A[nb[i]][nb[j]];
    charpoly4(A4, p);
    int st = quartic_roots(p, ev);
    if (st != OR_OK) return st;

    double K[6][6] = {{0.0}}, mu[6];
    for (int k = 0; k < 4; ++k) {
        double M[4][4], v[4];
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j) M[i][j] = A4[i][j] - (i == j ? ev[k] : 0.0);
        null_vector4(M, v);
        for (int i = 0; i < 4; ++i) K[nb[i]][k] = v[i];
        /* q_kt rows of (A6 - lam I) v = 0 */
        for (int t = 2; t <= 5; t += 3) {
            double sum = 0.0;
            for (int j = 0; j < 6; ++j)
                if (j != t) sum += A[t][j] * K[j][k];
            K[t][k] = sum / (ev[k] - A[t][t]);
        }
        mu[k] = ev[k];
    }
    K[2][4] = 1.0;
    mu[4] = u1;
    K[5][5] = 1.0;
    mu[5] = u2;

    double FL[6] = {q1L, q1L * q1L / h1L + 0.5 * g * h1L * h1L, q1L * t1L / h1L,
                    q2L, q2L * q2L / h2L + 0.5 * g * h2L * h2L, q2L * t2L / h2L};
    double FR[6] = {q1R, q1R * q1R / h1R + 0.5 * g * h1R * h1R, q1R * t1R / h1R,
                    q2R, q2R * q2R / h2R + 0.5 * g * h2R * h2R, q2R * t2R / h2R};
    double dW[6] = {h1R - h1L, q1R - q1L, t1R - t1L, h2R - h2L, q2R - q2L, t2R - t2L};
    double X[6];
    for (int i = 0; i < 6; ++i) {
        double BdW = 0.0;
        for (int j = 0; j < 6; ++j) BdW += B[i][j] * dW[j];
        X[i] = FR[i] - FL[i] - BdW - S[i] * (HR - HL);
    }
    double alpha[6];
    st = solve_n(6, K, X, alpha);
    if (st != OR_OK) return st;
    for (int i = 0; i < 6; ++i) phi[i] = FL[i];
    double m = 0.0;
    for (int k = 0; k < 6; ++k) {
        double w = 0.5 * (1.0 - sgn(mu[k]));
        for (int i = 0; i < 6; ++i) phi[i] += w * alpha[k] * K[i][k];
        m = fmax(m, fabs(mu[k]));
    }
    *speed = m;
    if (lam)
        for (int k = 0; k < 4; ++k) lam[k] = ev[k];
    return OR_OK;
}

/* Reflective wall, two layers: mirror ghost through the same flux, then the
 * mass (and hence transverse) fluxes set to exactly zero. */
int or_roe2_wall(const double *L, double g, double r, double *phi, double *speed)
{
    double Rg[7] = {L[0], -L[1], L[2], L[3], -L[4], L[5], L[6]};
    int st = or_roe2_edge(L, Rg, g, r, phi, speed, NULL);
    if (st != OR_OK) return st;
    phi[0] = 0.0;
    phi[2] = 0.0;
    phi[3] = 0.0;
    phi[5] = 0.0;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Cartesian grids, one layer (+ optional pollutant)                        */
/* ------------------------------------------------------------------------ */

static int check_state(int64_t n, int nv, double *const *W)
{
    for (int64_t i = 0; i < n; ++i) {
        for (int v = 0; v < nv; ++v)
            if (!isfinite(W[v][i])) return OR_NONFINITE;
        if (!(W[0][i] > 0.0)) return OR_DEPTH;
    }
    return OR_OK;
}

/* Runs nsteps steps in place.  State arrays of nx*ny cells, cell j*nx+i.
 * hc may be NULL (no pollutant).  dts[s] receives the step's dt. */
int or_run_cart(int nx, int ny, double dx, double dy, int periodic_x,
                int periodic_y, double g, double cfl, int nsteps,
                const double *z, double *h, double *qx, double *qy, double *hc,
                double *dts, int nthreads, int classical, int fix)
{
    int64_t N = (int64_t)nx * ny;
    double area = dx * dy;
    double *acc = malloc(sizeof(double) * 4 * N);
    double *dti = malloc(sizeof(double) * N);
    if (!acc || !dti) { free(acc); free(dti); return OR_NOMEM; }
    int status = OR_OK;
    if (nthreads < 1) nthreads = 1;

    for (int s = 0; s < nsteps && status == OR_OK; ++s) {
        int err = OR_OK;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(max : err)
        for (int64_t k = 0; k < N; ++k) {
            int i = (int)(k % nx), j = (int)(k / nx);
            /* sides: left, right, bottom, top with outward normals */
            const int di[4] = {-1, 1, 0, 0}, dj[4] = {0, 0, -1, 1};
            const double ex[4] = {-1.0, 1.0, 0.0, 0.0}, ey[4] = {0.0, 0.0, -1.0, 1.0};
            const double len[4] = {dy, dy, dx, dx};
            double a[4] = {0.0, 0.0, 0.0, 0.0}, S = 0.0;
            double cval = hc ? hc[k] : 0.0;
            for (int sd = 0; sd < 4; ++sd) {
                int ni = i + di[sd], nj = j + dj[sd];
                int wall = 0;
                if (ni < 0 || ni >= nx) {
                    if (periodic_x) ni = (ni + nx) % nx; else wall = 1;
                }
                if (nj < 0 || nj >= ny) {
                    if (periodic_y) nj = (nj + ny) % ny; else wall = 1;
                }
                double Lst[5] = {h[k], qx[k] * ex[sd] + qy[k] * ey[sd],
                                 -qx[k] * ey[sd] + qy[k] * ex[sd], cval, -z[k]};
                double phi[4], sp;
                int st;
                if (wall) {
                    st = or_roe1_wall(Lst, g, phi, &sp);
                } else {
                    int64_t m = (int64_t)nj * nx + ni;
                    double Rst[5] = {h[m], qx[m] * ex[sd] + qy[m] * ey[sd],
                                     -qx[m] * ey[sd] + qy[m] * ex[sd],
                                     hc ? hc[m] : 0.0, -z[m]};
                    st = classical ? roe1_classical(Lst, Rst, g, fix, phi, &sp)
                                   : roe1_ir(Lst, Rst, g, fix, phi, &sp);
                }
                if (st > err) err = st;
                /* back-rotation T^-1 and accumulation of |G| F^- */
                a[0] += len[sd] * phi[0];
                a[1] += len[sd] * (ex[sd] * phi[1] - ey[sd] * phi[2]);
                a[2] += len[sd] * (ey[sd] * phi[1] + ex[sd] * phi[2]);
                a[3] += len[sd] * phi[3];
                S += len[sd] * sp;
            }
            for (int v = 0; v < 4; ++v) acc[4 * k + v] = a[v];
            dti[k] = 2.0 * cfl * area / S;
        }
        if (err != OR_OK) { status = err; break; }
        double dt = INFINITY;
        for (int64_t k = 0; k < N; ++k) dt = fmin(dt, dti[k]);
        if (dts) dts[s] = dt;
        double f = dt / area;
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int64_t k = 0; k < N; ++k) {
            h[k] -= f * acc[4 * k + 0];
            qx[k] -= f * acc[4 * k + 1];
            qy[k] -= f * acc[4 * k + 2];
            if (hc) hc[k] -= f * acc[4 * k + 3];
        }
        double *W[4] = {h, qx, qy, hc};
        status = check_state(N, hc ? 4 : 3, W);
    }
    free(acc);
    free(dti);
    return status;
}

/* ------------------------------------------------------------------------ */
/* Triangle meshes                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t nb[3];       /* neighbour cell across local edge k, or -1 (wall) */
    double ex[3], ey[3]; /* outward unit normal of local edge k              */
    double len[3];       /* length of local edge k                           */
    double area;
} or_tri_cell;

typedef struct {
    int64_t lo, hi, cell;
    int k;
} or_edge_key;

static int cmp_edge_key(const void *pa, const void *pb)
{
    const or_edge_key *a = pa, *b = pb;
    if (a->lo != b->lo) return a->lo < b->lo ? -1 : 1;
    if (a->hi != b->hi) return a->hi < b->hi ? -1 : 1;
    if (a->cell != b->cell) return a->cell < b->cell ? -1 : 1;
    return a->k - b->k;
}

/* Geometry of every cell: edge k joins corners k and k+1 (counter-
 * clockwise), so the outward normal of the edge vector (dx, dy) is
 * (dy, -dx)/len. */
static int build_tri_cells(int64_t nnodes, const double *xy, int64_t ncells,
                           const int32_t *tri, or_tri_cell *cells)
{
    for (int64_t t = 0; t < ncells; ++t) {
        int64_t v[3];
        for (int k = 0; k < 3; ++k) {
            v[k] = tri[3 * t + k];
            if (v[k] < 0 || v[k] >= nnodes) return OR_BADMESH;
        }
        double x0 = xy[2 * v[0]], y0 = xy[2 * v[0] + 1];
        double x1 = xy[2 * v[1]], y1 = xy[2 * v[1] + 1];
        double x2 = xy[2 * v[2]], y2 = xy[2 * v[2] + 1];
        double area = 0.5 * ((x1 - x0) * (y2 - y0) - (x2 - x0) * (y1 - y0));
        if (!(area > 0.0)) return OR_BADMESH;
        cells[t].area = area;
        for (int k = 0; k < 3; ++k) {
            int64_t a = v[k], b = v[(k + 1) % 3];
            double ddx = xy[2 * b] - xy[2 * a], ddy = xy[2 * b + 1] - xy[2 * a + 1];
            double len = sqrt(ddx * ddx + ddy * ddy);
            cells[t].len[k] = len;
            cells[t].ex[k] = ddy / len;
            cells[t].ey[k] = -ddx / len;
            cells[t].nb[k] = -1;
        }
    }
    or_edge_key *keys = malloc(sizeof(or_edge_key) * 3 * ncells);
    if (!keys) return OR_NOMEM;
    for (int64_t t = 0; t < ncells; ++t)
        for (int k = 0; k < 3; ++k) {
            int64_t a = tri[3 * t + k], b = tri[3 * t + (k + 1) % 3];
            or_edge_key *e = &keys[3 * t + k];
            e->lo = a < b ? a : b;
            e->hi = a < b ? b : a;
            e->cell = t;
            e->k = k;
        }
    qsort(keys, 3 * ncells, sizeof(or_edge_key), cmp_edge_key);
    int status = OR_OK;
    for (int64_t i = 0; i < 3 * ncells;) {
        int64_t j = i + 1;
        while (j < 3 * ncells && keys[j].lo == keys[i].lo && keys[j].hi == keys[i].hi) ++j;
        if (j - i > 2) { status = OR_BADMESH; break; }
        if (j - i == 2) {
            cells[keys[i].cell].nb[keys[i].k] = keys[i + 1].cell;
            cells[keys[i + 1].cell].nb[keys[i + 1].k] = keys[i].cell;
        }
        i = j;
    }
    free(keys);
    return status;
}

/* One layer on triangles; hc may be NULL. */
int or_run_tri(int64_t nnodes, const double *xy, int64_t ncells,
               const int32_t *tri, double g, double cfl, int nsteps,
               const double *z, double *h, double *qx, double *qy, double *hc,
               double *dts, int nthreads, int classical, int fix)
{
    or_tri_cell *cells = malloc(sizeof(or_tri_cell) * ncells);
    double *acc = malloc(sizeof(double) * 4 * ncells);
    double *dti = malloc(sizeof(double) * ncells);
    if (!cells || !acc || !dti) { free(cells); free(acc); free(dti); return OR_NOMEM; }
    int status = build_tri_cells(nnodes, xy, ncells, tri, cells);
    if (nthreads < 1) nthreads = 1;

    for (int s = 0; s < nsteps && status == OR_OK; ++s) {
        int err = OR_OK;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(max : err)
        for (int64_t t = 0; t < ncells; ++t) {
            const or_tri_cell *C = &cells[t];
            double a[4] = {0.0, 0.0, 0.0, 0.0}, S = 0.0;
            for (int k = 0; k < 3; ++k) {
                double ex = C->ex[k], ey = C->ey[k];
                double Lst[5] = {h[t], qx[t] * ex + qy[t] * ey, -qx[t] * ey + qy[t] * ex,
                                 hc ? hc[t] : 0.0, -z[t]};
                double phi[4], sp;
                int st;
                int64_t m = C->nb[k];
                if (m < 0) {
                    st = or_roe1_wall(Lst, g, phi, &sp);
                } else {
                    double Rst[5] = {h[m], qx[m] * ex + qy[m] * ey, -qx[m] * ey + qy[m] * ex,
                                     hc ? hc[m] : 0.0, -z[m]};
                    st = classical ? roe1_classical(Lst, Rst, g, fix, phi, &sp)
                                   : roe1_ir(Lst, Rst, g, fix, phi, &sp);
                }
                if (st > err) err = st;
                a[0] += C->len[k] * phi[0];
                a[1] += C->len[k] * (ex * phi[1] - ey * phi[2]);
                a[2] += C->len[k] * (ey * phi[1] + ex * phi[2]);
                a[3] += C->len[k] * phi[3];
                S += C->len[k] * sp;
            }
            for (int v = 0; v < 4; ++v) acc[4 * t + v] = a[v];
            dti[t] = 2.0 * cfl * C->area / S;
        }
        if (err != OR_OK) { status = err; break; }
        double dt = INFINITY;
        for (int64_t t = 0; t < ncells; ++t) dt = fmin(dt, dti[t]);
        if (dts) dts[s] = dt;
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int64_t t = 0; t < ncells; ++t) {
            double f = dt / cells[t].area;
            h[t] -= f * acc[4 * t + 0];
            qx[t] -= f * acc[4 * t + 1];
            qy[t] -= f * acc[4 * t + 2];
            if (hc) hc[t] -= f * acc[4 * t + 3];
        }
        double *W[4] = {h, qx, qy, hc};
        status = check_state(ncells, hc ? 4 : 3, W);
    }
    free(cells);
    free(acc);
    free(dti);
    return status;
}

/* Two layers on triangles.  W = h1, q1x, q1y, h2, q2x, q2y. */
int or_run_tri2(int64_t nnodes, const double *xy, int64_t ncells,
                const int32_t *tri, double g, double r, double cfl, int nsteps,
                const double *z, double *h1, double *q1x, double *q1y,
                double *h2, double *q2x, double *q2y, double *dts, int nthreads,
                int classical)
{
    or_tri_cell *cells = malloc(sizeof(or_tri_cell) * ncells);
    double *acc = malloc(sizeof(double) * 6 * ncells);
    double *dti = malloc(sizeof(double) * ncells);
    if (!cells || !acc || !dti) { free(cells); free(acc); free(dti); return OR_NOMEM; }
    int status = build_tri_cells(nnodes, xy, ncells, tri, cells);
    if (nthreads < 1) nthreads = 1;
    double *W[6] = {h1, q1x, q1y, h2, q2x, q2y};

    for (int s = 0; s < nsteps && status == OR_OK; ++s) {
        int err = OR_OK;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(max : err)
        for (int64_t t = 0; t < ncells; ++t) {
            const or_tri_cell *C = &cells[t];
            double a[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0}, S = 0.0;
            for (int k = 0; k < 3; ++k) {
                double ex = C->ex[k], ey = C->ey[k];
                double Lst[7] = {h1[t], q1x[t] * ex + q1y[t] * ey, -q1x[t] * ey + q1y[t] * ex,
                                 h2[t], q2x[t] * ex + q2y[t] * ey, -q2x[t] * ey + q2y[t] * ex,
                                 -z[t]};
                double phi[6], sp;
                int st;
                int64_t m = C->nb[k];
                if (m < 0) {
                    st = or_roe2_wall(Lst, g, r, phi, &sp);
                } else {
                    double Rst[7] = {h1[m], q1x[m] * ex + q1y[m] * ey, -q1x[m] * ey + q1y[m] * ex,
                                     h2[m], q2x[m] * ex + q2y[m] * ey, -q2x[m] * ey + q2y[m] * ex,
                                     -z[m]};
                    st = classical ? or_roe2c_edge(Lst, Rst, g, r, phi, &sp, NULL)
                                   : or_roe2_edge(Lst, Rst, g, r, phi, &sp, NULL);
                }
                if (st > err) err = st;
                if (st != OR_OK) continue;
                for (int l = 0; l < 2; ++l) {
                    a[3 * l + 0] += C->len[k] * phi[3 * l + 0];
                    a[3 * l + 1] += C->len[k] * (ex * phi[3 * l + 1] - ey * phi[3 * l + 2]);
                    a[3 * l + 2] += C->len[k] * (ey * phi[3 * l + 1] + ex * phi[3 * l + 2]);
                }
                S += C->len[k] * sp;
            }
            for (int v = 0; v < 6; ++v) acc[6 * t + v] = a[v];
            dti[t] = 2.0 * cfl * C->area / S;
        }
        if (err != OR_OK) { status = err; break; }
        double dt = INFINITY;
        for (int64_t t = 0; t < ncells; ++t) dt = fmin(dt, dti[t]);
        if (dts) dts[s] = dt;
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int64_t t = 0; t < ncells; ++t) {
            double f = dt / cells[t].area;
            for (int v = 0; v < 6; ++v) W[v][t] -= f * acc[6 * t + v];
        }
        status = check_state(ncells, 6, W);
        if (status == OR_OK)
            for (int64_t t = 0; t < ncells; ++t)
                if (!(h2[t] > 0.0)) { status = OR_DEPTH; break; }
    }
    free(cells);
    free(acc);
    free(dti);
    return status;
}

/* Geometry export for tests: per cell neighbours, outward normals, lengths
 * and area, as the oracle derives them. */
int or_tri_geometry(int64_t nnodes, const double *xy, int64_t ncells,
                    const int32_t *tri, int64_t *nb, double *ex, double *ey,
                    double *len, double *area)
{
    or_tri_cell *cells = malloc(sizeof(or_tri_cell) * ncells);
    if (!cells) return OR_NOMEM;
    int st = build_tri_cells(nnodes, xy, ncells, tri, cells);
    if (st == OR_OK)
        for (int64_t t = 0; t < ncells; ++t) {
            for (int k = 0; k < 3; ++k) {
                nb[3 * t + k] = cells[t].nb[k];
                ex[3 * t + k] = cells[t].ex[k];
                ey[3 * t + k] = cells[t].ey[k];
                len[3 * t + k] = cells[t].len[k];
            }
            area[t] = cells[t].area;
        }
    free(cells);
    return st;
}
