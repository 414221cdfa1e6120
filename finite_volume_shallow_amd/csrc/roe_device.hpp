// Device-side Roe edge fluxes in fluctuation form.
//
// The IR-Roe flux of [IR] Sec. 2.2 (de la Asuncion et al., "An MPI-CUDA
// implementation of an improved Roe method for two-layer shallow water
// systems") is, in the frame of the edge normal eta (pointing from cell a to
// cell b),
//     Phi^- = F(W_a) + P^- X,   X = F(W_b) - F(W_a) - B dW - S dH,
//     P^- = 1/2 K (I - sgn D) K^-1,
// plus the transverse momentum carried by the mass flux and upwinded by its
// sign (step 3).  Cell a's update uses |G| T^-1 Phi^-; cell b's (outward
// normal -eta) uses -|G| T^-1 Phi^+ with Phi^+ = Phi^- + B dW + S dH.
// Because sum_j |G_ij| eta_ij = 0 on a closed cell, the physical flux of the
// cell itself drops out of the sum of Eq. (4), so each edge only has to hand
// its two cells the fluctuations (in the frame of eta)
//     a:  Phi^- - F(W_a)           =  P^- X
//     b:  -(Phi^+ - F(W_b))        =  X - P^- X      (Phi^+ = F(W_b) - X + P^- X)
// plus the matching transverse-momentum and pollutant parts; the update is
// W_i -= dt/|V_i| sum |G| T^-1 (fluctuation).  This form carries only
// differences, which keeps the float32 path accurate (no cancellation of
// the large hydrostatic terms).
//
// The pollutant flux is a passive scalar carried by the mass flux and
// upwinded like the transverse momentum ([MG] Vinas et al., "A multi-GPU
// shallow-water simulation with transport of contaminants": a transport
// equation on top of the one-layer model).
//
// Reflective walls are the mirror-ghost Riemann problem with the mass,
// transverse and pollutant fluxes set to exactly zero; the normal-momentum
// fluctuation of that problem is sqrt(g h) q_n.
#pragma once

#include <hip/hip_runtime.h>

#include "fastmath.hpp"

namespace swe {

template <typename T> __device__ __forceinline__ T rcp(T x) { return FM<T>::rcp(x); }


// sgn-weights 1/2 (1 - sgn(lambda)) with sgn(0) = 0, branch-free:
// clamp(1/2 - lambda 2^K, 0, 1) is exactly 1, 0, 1/2 for lambda < 0, > 0,
// = 0 whenever |lambda| >= 2^-(K+1) or lambda = 0.  A wave speed is a sum
// u +- c with c = sqrt(g h) > 0, so a nonzero one is at least an ulp of c,
// far above 2^-101 (float) or 2^-601 (double); the product overflowing to
// +-inf clamps correctly.
template <typename T> __device__ __forceinline__ T wminus(T lam);
template <> __device__ __forceinline__ float wminus(float lam)
{
    return __builtin_amdgcn_fmed3f(__builtin_fmaf(lam, -0x1p100f, 0.5f), 0.0f, 1.0f);
}
template <> __device__ __forceinline__ double wminus(double lam)
{
    return fmin(fmax(__builtin_fma(lam, -0x1p600, 0.5), 0.0), 1.0);
}

// Flux variants of the one-layer edge: IR-Roe, the classical Roe flux of
// the whole edge system, and each with the Harten-Hyman entropy fix.
enum : int { FLUX_IR = 0, FLUX_ROE = 1, FLUX_IR_HH = 2, FLUX_ROE_HH = 3 };
__host__ __device__ constexpr bool flux_classical(int fx) { return fx == FLUX_ROE || fx == FLUX_ROE_HH; }
__host__ __device__ constexpr bool flux_hh(int fx) { return fx == FLUX_IR_HH || fx == FLUX_ROE_HH; }

// Harten-Hyman entropy fix of the 2x2 Roe solution ([IR] Sec. 2.2 names the
// fix of its ref. 25).  b = K^-1 (W_b - W_a) are the waves' state jumps and
// W* = W_a + b1 r1 the state between them; a wave whose characteristic
// speed is < 0 on its left state and > 0 on its right one (a transonic
// rarefaction) is split into a part moving left at the left speed and one
// moving right at the right speed, carrying the fraction
// (lam_right - lam~)/(lam_right - lam_left) to the left, so its left-going
// flux jump min(lam~, 0) b r becomes lam_left (lam_right - lam~) /
// (lam_right - lam_left) b r.  (pm0, pm1) is the left-going flux jump P^- X;
// the source part of each wave is untouched.  i2c = 1 / (lam2 - lam1).
template <typename T>
__device__ __forceinline__ void hh_fix(T hL, T qL, T uL, T hR, T qR, T uR, T lam1, T lam2, T i2c, T g, T &pm0,
                                       T &pm1)
{
    const T dh = hR - hL, dq = qR - qL;
    const T b1 = (lam2 * dh - dq) * i2c;
    const T b2 = (dq - lam1 * dh) * i2c;
    const T hs = hL + b1, qs = qL + b1 * lam1;
    // a wave can only be transonic if W* is supercritical (u* - c* > 0 for
    // the first, u* + c* < 0 for the second): q*^2 > g h*^3, no root needed
    if (hs > T(0) && qs * qs > g * hs * hs * hs) {
        const T us = qs * FM<T>::rcp(hs), cs = FM<T>::sqrt(g * hs);
        const T l1L = uL - FM<T>::sqrt(g * hL), l1R = us - cs;
        const T l2L = us + cs, l2R = uR + FM<T>::sqrt(g * hR);
        T k1 = T(0), k2 = T(0);
        if (l1L < T(0) && l1R > T(0)) k1 = (l1L * (l1R - lam1) * FM<T>::rcp(l1R - l1L) - fmin(lam1, T(0))) * b1;
        if (l2L < T(0) && l2R > T(0)) k2 = (l2L * (l2R - lam2) * FM<T>::rcp(l2R - l2L) - fmin(lam2, T(0))) * b2;
        pm0 += k1 + k2;
        pm1 += k1 * lam1 + k2 * lam2;
    }
}

// One-layer interior edge.  Inputs are edge-frame states: depth h, normal
// discharge qn, transverse discharge qt, pollutant hc, bed z.
// Output: fluctuations for side a (da*) and side b (db*), in the edge frame,
// and the largest |eigenvalue| of the Roe matrix (|u| + c).
template <typename T, bool TRACER> struct Flux1 {
    T am, an, at, ac;
    T bm, bn, bt, bc;
    T speed;
};

// As roe1_interior, with sqrt(h) and 1/h of both cells supplied.
//
// FX = FLUX_ROE selects the classical Roe flux of the whole edge system
// (h, qn, qt, hc): its Roe matrix adds to the 2x2 block two contact waves of
// speed ubar, with eigenvectors e_qt and e_hc, while the acoustic
// eigenvectors carry the Roe averages vbar, Cbar (sqrt(h)-weighted, like
// ubar) in those rows.  With alpha_t = X_t - vbar X_0 and
// alpha_c = X_c - Cbar X_0, the side-a fluctuation of those rows is
// vbar (P^- X)_0 + w(ubar) alpha_t, and the same with Cbar; mass and normal
// momentum are those of the IR-Roe flux.
template <typename T, bool TRACER, int FX = FLUX_IR>
__device__ __forceinline__ Flux1<T, TRACER> roe1_pre(T hL, T sL, T ihL, T qnL, T qtL, T cL, T zL, T hR, T sR,
                                                      T ihR, T qnR, T qtR, T cR, T zR, T g)
{
    Flux1<T, TRACER> o;
    const T uL = qnL * ihL, uR = qnR * ihR;
    const T isum = rcp(sL + sR);
    const T ubar = (sL * uL + sR * uR) * isum;
    // classical flux: the contact waves' Roe averages and jumps are formed
    // here, so that their inputs (the transverse velocities and sqrt(h)
    // weights) are no longer needed during the 2x2 part
    T vbar = T(0), Xt = T(0), cbar = T(0), Xc = T(0);
    if (flux_classical(FX)) {
        const T utL = qtL * ihL, utR = qtR * ihR;
        vbar = (sL * utL + sR * utR) * isum;
        Xt = qnR * utR - qnL * utL;
        if (TRACER) {
            const T ccL = cL * ihL, ccR = cR * ihR;
            cbar = (sL * ccL + sR * ccR) * isum;
            Xc = qnR * ccR - qnL * ccL;
        }
    }
    const T hbar = T(0.5) * (hL + hR);
    const T c2 = g * hbar;
    const T irc = FM<T>::rsq(c2);
    const T c = c2 * irc;
    const T lam1 = ubar - c, lam2 = ubar + c;
    // X = (dqn, d(qn u) + g hbar (dh + dz)); g/2 (hR^2 - hL^2) = g hbar dh.
    const T X0 = qnR - qnL;
    const T X1 = (qnR * uR - qnL * uL) + c2 * ((hR - hL) + (zR - zL));
    const T i2c = T(0.5) * irc;
    const T a1 = (lam2 * X0 - X1) * i2c;
    const T a2 = (X1 - lam1 * X0) * i2c;
    const T w1 = wminus(lam1), w2 = wminus(lam2);
    T pm0 = w1 * a1 + w2 * a2;
    T pm1 = w1 * a1 * lam1 + w2 * a2 * lam2;
    if (flux_hh(FX)) hh_fix(hL, qnL, uL, hR, qnR, uR, lam1, lam2, i2c, g, pm0, pm1);
    o.am = pm0;
    o.an = pm1;
    o.bm = X0 - pm0;
    o.bn = X1 - pm1;
    if (flux_classical(FX)) {
        const T wu = wminus(ubar);
        o.at = vbar * pm0 + wu * (Xt - vbar * X0);
        o.bt = Xt - o.at;
        if (TRACER) {
            o.ac = cbar * pm0 + wu * (Xc - cbar * X0);
            o.bc = Xc - o.ac;
        } else {
            o.ac = T(0);
            o.bc = T(0);
        }
        o.speed = fabs(ubar) + c;
        return o;
    }
    const T utL = qtL * ihL, utR = qtR * ihR;
    const T phi0 = qnL + pm0; // mass flux through the edge
    if (phi0 > T(0)) {
        o.at = pm0 * utL;                    // phi0 utL - qnL utL
        o.bt = qnR * utR - phi0 * utL;       // -(phi0 utL - qnR utR)
    } else {
        o.at = phi0 * utR - qnL * utL;
        o.bt = (X0 - pm0) * utR;             // -(phi0 - qnR) utR
    }
    if (TRACER) {
        const T ccL = cL * ihL, ccR = cR * ihR;
        if (phi0 > T(0)) {
            o.ac = pm0 * ccL;
            o.bc = qnR * ccR - phi0 * ccL;
        } else {
            o.ac = phi0 * ccR - qnL * ccL;
            o.bc = (X0 - pm0) * ccR;
        }
    } else {
        o.ac = T(0);
        o.bc = T(0);
    }
    o.speed = fabs(ubar) + c;
    return o;
}

template <typename T, bool TRACER, int FX = FLUX_IR>
__device__ __forceinline__ Flux1<T, TRACER> roe1_interior(T hL, T qnL, T qtL, T cL, T zL,
                                                           T hR, T qnR, T qtR, T cR, T zR, T g)
{
    const T rL = FM<T>::rsq(hL), rR = FM<T>::rsq(hR);
    return roe1_pre<T, TRACER, FX>(hL, hL * rL, rL * rL, qnL, qtL, cL, zL, hR, hR * rR, rR * rR, qnR, qtR, cR, zR, g);
}

// One-layer reflective wall seen from side a.
template <typename T, bool TRACER>
__device__ __forceinline__ Flux1<T, TRACER> roe1_wall(T h, T qn, T qt, T hc, T g)
{
    Flux1<T, TRACER> o;
    const T c = FM<T>::sqrt(g * h);
    const T ih = rcp(h);
    o.am = -qn;
    o.an = c * qn;
    o.at = -qn * qt * ih;
    o.ac = TRACER ? -qn * hc * ih : T(0);
    o.bm = o.bn = o.bt = o.bc = T(0);
    o.speed = c;
    return o;
}

// ---------------------------------------------------------------------------
// Two layers.  The 4x4 Roe matrix of [IR] Sec. 2.2 on (h1, q1, h2, q2):
//   A = [[0, 1, 0, 0], [c1^2 - u1^2, 2 u1, c1^2, 0], [0, 0, 0, 1],
//        [r c2^2, 0, c2^2 - u2^2, 2 u2]],   c_k^2 = g hbar_k,
// (r sits in the lower-layer row: -r g h2 d(h1) is the lower layer's
// coupling term).  Its eigenvalues are the roots of
//   Q(l) = ((l - u1)^2 - c1^2) ((l - u2)^2 - c2^2) - r c1^2 c2^2,
// right eigenvectors (1, l, s, l s) with s = ((l - u1)^2 - c1^2) / c1^2 and
// left eigenvectors ((l - 2 u1) t, t, (l - 2 u2) c1^2, c1^2) with
// t = (l - u2)^2 - c2^2; the product of a left and its right eigenvector is
// Q'(l).  So alpha_k = l_k . X / Q'(l_k) needs no matrix inversion.
//
// Roots: the two outer roots by Newton, the two inner roots from the
// deflated quadratic, each polished by one Newton step on the factored form
// of Q.  A negative discriminant of the deflated quadratic means complex
// speeds: the state is flagged non-hyperbolic.
//
// Newton starts for the outer roots.  Write P for the product term alone
// (no coupling): its roots are d_k -/+ c_k, and Q = P - r c1^2 c2^2 < P,
// so the largest root of Q lies above the largest root p4 of P, where P
// (and Q) is already increasing and convex; Newton started anywhere at or
// beyond p4 converges to it monotonically after at most one overshoot.
// The start is the outer root of the motionless pair (d1 = d2 = 0, a
// biquadratic: mu^2 = (c1^2 + c2^2 + sqrt((c1^2 - c2^2)^2 + 4 r c1^2 c2^2))/2)
// shifted by the c^2-weighted mean of d1, d2, raised to p4 if below it;
// mirrored for the smallest root.  That start is within a few 1e-5 of the
// root for the flows of interest, so one or two steps suffice.  Iteration
// stops once a step is below sqrt-epsilon of the root: Newton's quadratic
// convergence leaves the iterate after such a step accurate to rounding.
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------

template <typename T> struct Flux2 {
    T a[6]; // side a: h1, q1n, q1t, h2, q2n, q2t
    T b[6]; // side b
    T speed;
    bool nonhyp;
};

template <typename T>
__device__ __forceinline__ T quartic_q(T mu, T d1, T d2, T c1, T c2, T rc)
{
    const T e1 = mu - d1, e2 = mu - d2;
    return (e1 * e1 - c1) * (e2 * e2 - c2) - rc;
}

template <typename T>
__device__ __forceinline__ T quartic_dq(T mu, T d1, T d2, T c1, T c2)
{
    const T e1 = mu - d1, e2 = mu - d2;
    return T(2) * (e1 * (e2 * e2 - c2) + e2 * (e1 * e1 - c1));
}

template <typename T> struct NewtonStop;
template <> struct NewtonStop<double> { static constexpr double v = 1e-8; };
template <> struct NewtonStop<float> { static constexpr float v = 1e-4f; };

// square root good enough for a starting point (hardware estimate, 0 for 0)
template <typename T> __device__ __forceinline__ T sqrt_start(T x)
{
    return x > T(0) ? x * FM<T>::rsq_est(x) : T(0);
}

// Largest (hi) and smallest (lo) root of Q in the shifted variable.
template <typename T>
__device__ __forceinline__ void outer_roots(T d1, T d2, T c1, T c2, T rc, T &hi, T &lo)
{
    const T s1 = sqrt_start(c1), s2 = sqrt_start(c2);
    const T dc = c1 - c2;
    const T w = sqrt_start(T(0.5) * ((c1 + c2) + sqrt_start(dc * dc + T(4) * rc)));
    const T um = (d1 * c1 + d2 * c2) * rcp(c1 + c2);
    // p4 / p1 from estimated square roots: moved out by a margin that covers
    // their error (and keeps Q' > 0 off a double root of P)
    const T mg = T(1e-4) * (s1 + s2);
    hi = fmax(um + w, fmax(d1 + s1, d2 + s2) + mg);
    lo = fmin(um - w, fmin(d1 - s1, d2 - s2) - mg);
    bool dh = false, dl = false;
    for (int it = 0; it < 40; ++it) {
        const T fh = quartic_q(hi, d1, d2, c1, c2, rc), gh = quartic_dq(hi, d1, d2, c1, c2);
        const T fl = quartic_q(lo, d1, d2, c1, c2, rc), gl = quartic_dq(lo, d1, d2, c1, c2);
        const T sh = fh == T(0) ? T(0) : fh * FM<T>::rcp_est(gh);
        const T sl = fl == T(0) ? T(0) : fl * FM<T>::rcp_est(gl);
        if (!dh) hi -= sh;
        if (!dl) lo -= sl;
        dh = dh || !(fabs(sh) > NewtonStop<T>::v * fabs(hi));
        dl = dl || !(fabs(sl) > NewtonStop<T>::v * fabs(lo));
        if (dh && dl) break;
    }
}

template <typename T>
__device__ __forceinline__ T newton_polish(T mu, T d1, T d2, T c1, T c2, T rc)
{
    const T df = quartic_dq(mu, d1, d2, c1, c2);
    return df != T(0) ? mu - quartic_q(mu, d1, d2, c1, c2, rc) * FM<T>::rcp_est(df) : mu;
}

// L/R: h1, q1n, q1t, h2, q2n, q2t (edge frame), z; pL/pR: sqrt(h1), 1/h1,
// sqrt(h2), 1/h2 of each cell.
//
// CL selects the classical Roe flux of the whole 6x6 system: each layer's
// transverse momentum row (-u_k v_k, v_k, u_k) adds a contact wave of speed
// u_k with eigenvector e_{q_kt}, and completes every eigenvector of A_ij
// with v_k times its h_k component.  So alpha of that contact wave is
// X_kt - v_k X_hk and the side-a transverse fluctuation is
// v_k (P^- X)_hk + w(u_k) (X_kt - v_k X_hk); the normal rows are unchanged.
template <typename T, bool CL = false>
__device__ __forceinline__ Flux2<T> roe2_pre(const T *L, const T *pL, T zL, const T *R, const T *pR, T zR, T g,
                                             T r)
{
    Flux2<T> o;
    o.nonhyp = false;
    const T h1L = L[0], q1L = L[1], t1L = L[2], h2L = L[3], q2L = L[4], t2L = L[5];
    const T h1R = R[0], q1R = R[1], t1R = R[2], h2R = R[3], q2R = R[4], t2R = R[5];
    const T i1L = pL[1], i1R = pR[1], i2L = pL[3], i2R = pR[3];
    const T v1L = q1L * i1L, v1R = q1R * i1R, v2L = q2L * i2L, v2R = q2R * i2R;
    const T s1L = pL[0], s1R = pR[0], s2L = pL[2], s2R = pR[2];
    const T is1 = rcp(s1L + s1R), is2 = rcp(s2L + s2R);
    const T u1 = (s1L * v1L + s1R * v1R) * is1;
    const T u2 = (s2L * v2L + s2R * v2R) * is2;
    const T c1 = g * T(0.5) * (h1L + h1R); // c1^2
    const T c2 = g * T(0.5) * (h2L + h2R); // c2^2
    const T rc = r * c1 * c2;

    // X = dF - B dW - S dH with H = -z, written with g/2 d(h^2) = g hbar dh
    const T dh1 = h1R - h1L, dh2 = h2R - h2L, dz = zR - zL;
    T X[4];
    X[0] = q1R - q1L;
    X[1] = (q1R * v1R - q1L * v1L) + c1 * ((dh1 + dh2) + dz);
    X[2] = q2R - q2L;
    X[3] = (q2R * v2R - q2L * v2L) + c2 * ((dh2 + r * dh1) + dz);

    // eigenvalues in the shifted variable mu = lambda - m
    const T m = T(0.5) * (u1 + u2);
    const T d1 = u1 - m, d2 = u2 - m;
    T muhi, mulo;
    outer_roots(d1, d2, c1, c2, rc, muhi, mulo);
    // Q(mu) = mu^4 + a3 mu^3 + a2 mu^2 + a1 mu + a0; divide by (mu-muhi)(mu-mulo)
    const T p1 = d1 * d1 - c1, p2 = d2 * d2 - c2;
    const T a3 = T(-2) * (d1 + d2);
    const T a2 = p1 + p2 + T(4) * d1 * d2;
    const T sum = muhi + mulo, prod = muhi * mulo;
    const T b1 = a3 + sum;
    const T b0 = a2 + sum * b1 - prod;
    T disc = b1 * b1 - T(4) * b0;
    if (disc < T(0)) {
        o.nonhyp = true;
        disc = T(0);
    }
    const T sq = disc > T(0) ? FM<T>::sqrt(disc) : T(0);
    T mid1 = T(-0.5) * (b1 + sq), mid2 = T(-0.5) * (b1 - sq);
    mid1 = newton_polish(mid1, d1, d2, c1, c2, rc);
    mid2 = newton_polish(mid2, d1, d2, c1, c2, rc);

    T lam[4] = {mulo + m, mid1 + m, mid2 + m, muhi + m};
    T PX[4] = {T(0), T(0), T(0), T(0)};
    T smax = T(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const T l = lam[k];
        const T e1 = l - u1, e2 = l - u2;
        const T rho = e1 * e1 - c1;     // c1^2 s
        const T tau = e2 * e2 - c2;
        const T dq = T(2) * (tau * e1 + rho * e2);
        const T lx = (l - T(2) * u1) * tau * X[0] + tau * X[1] + (l - T(2) * u2) * c1 * X[2] + c1 * X[3];
        const T alpha = lx * rcp(dq);
        const T w = wminus(l);
        const T sgm = rho * rcp(c1);
        PX[0] += w * alpha;
        PX[1] += w * alpha * l;
        PX[2] += w * alpha * sgm;
        PX[3] += w * alpha * l * sgm;
        smax = fmax(smax, fabs(l));
    }
    o.speed = smax;
    o.a[0] = PX[0];
    o.a[1] = PX[1];
    o.a[3] = PX[2];
    o.a[4] = PX[3];
    o.b[0] = X[0] - PX[0];
    o.b[1] = X[1] - PX[1];
    o.b[3] = X[2] - PX[2];
    o.b[4] = X[3] - PX[3];
    const T w1L = t1L * i1L, w1R = t1R * i1R, w2L = t2L * i2L, w2R = t2R * i2R;
    if (CL) { // contact waves of the layers' Roe velocities
        const T vb1 = (s1L * w1L + s1R * w1R) * is1, vb2 = (s2L * w2L + s2R * w2R) * is2;
        const T Xt1 = q1R * w1R - q1L * w1L, Xt2 = q2R * w2R - q2L * w2L;
        o.a[2] = vb1 * PX[0] + wminus(u1) * (Xt1 - vb1 * X[0]);
        o.a[5] = vb2 * PX[2] + wminus(u2) * (Xt2 - vb2 * X[2]);
        o.b[2] = Xt1 - o.a[2];
        o.b[5] = Xt2 - o.a[5];
        return o;
    }
    // transverse momentum of each layer, upwinded by that layer's mass flux
    const T phi1 = q1L + PX[0], phi2 = q2L + PX[2];
    if (phi1 > T(0)) {
        o.a[2] = PX[0] * w1L;
        o.b[2] = q1R * w1R - phi1 * w1L;
    } else {
        o.a[2] = phi1 * w1R - q1L * w1L;
        o.b[2] = (X[0] - PX[0]) * w1R;
    }
    if (phi2 > T(0)) {
        o.a[5] = PX[2] * w2L;
        o.b[5] = q2R * w2R - phi2 * w2L;
    } else {
        o.a[5] = phi2 * w2R - q2L * w2L;
        o.b[5] = (X[2] - PX[2]) * w2R;
    }
    return o;
}

// Per-cell sqrt(h_k), 1/h_k of a two-layer state.
template <typename T> __device__ __forceinline__ void roe2_cellpre(const T *W, T *p)
{
    const T r1 = FM<T>::rsq(W[0]), r2 = FM<T>::rsq(W[3]);
    p[0] = W[0] * r1;
    p[1] = r1 * r1;
    p[2] = W[3] * r2;
    p[3] = r2 * r2;
}

template <typename T, bool CL = false>
__device__ __forceinline__ Flux2<T> roe2_interior(const T *L, T zL, const T *R, T zR, T g, T r)
{
    T pL[4], pR[4];
    roe2_cellpre(L, pL);
    roe2_cellpre(R, pR);
    return roe2_pre<T, CL>(L, pL, zL, R, pR, zR, g, r);
}

// Two-layer reflective wall seen from side a: the mirror ghost through the
// 4x4 flux, then both mass fluxes (hence the transverse fluxes) set to zero.
template <typename T>
__device__ __forceinline__ Flux2<T> roe2_wall_pre(const T *L, const T *pL, T z, T g, T r)
{
    const T G[6] = {L[0], -L[1], L[2], L[3], -L[4], L[5]};
    Flux2<T> o = roe2_pre<T>(L, pL, z, G, pL, z, g, r);
    o.a[0] = -L[1];
    o.a[3] = -L[4];
    o.a[2] = -L[1] * L[2] * rcp(L[0]);
    o.a[5] = -L[4] * L[5] * rcp(L[3]);
#pragma unroll
    for (int v = 0; v < 6; ++v) o.b[v] = T(0);
    return o;
}

template <typename T> __device__ __forceinline__ Flux2<T> roe2_wall(const T *L, T z, T g, T r)
{
    T p[4];
    roe2_cellpre(L, p);
    return roe2_wall_pre<T>(L, p, z, g, r);
}

} // namespace swe
