"""Edge-level pins of the oracle's Roe fluxes.

The oracle's one-layer flux uses the 2x2 closed form and its two-layer flux
uses Faddeev-LeVerrier + Durand-Kerner + adjugate eigenvectors + Gaussian
elimination.  Here both are checked against a generic library eigen-
decomposition of the Roe matrix A_ij as the IR-Roe paper defines it
(Sec. 2.2, with the density ratio r in the lower-layer row), against closed
forms, and against the jump conditions that a path-conservative scheme must
satisfy: the flux seen from the two sides of an edge differs exactly by the
non-conservative products B_ij dW + S_ij dH.
"""
import math

import numpy as np
import pytest

import oracle

G = 9.81


def _roe_avg(hL, qL, hR, qR):
    sL, sR = math.sqrt(hL), math.sqrt(hR)
    return (sL * qL / hL + sR * qR / hR) / (sL + sR), 0.5 * (hL + hR)


def _pminus(A):
    lam, K = np.linalg.eig(A)
    lam = lam.real
    K = K.real
    return K @ np.diag(0.5 * (1.0 - np.sign(lam))) @ np.linalg.inv(K), lam


def _flip(state, idx):
    s = np.array(state, dtype=float)
    s[list(idx)] *= -1.0
    return s


# --------------------------------------------------------------- one layer

def _random_states1(rng, n):
    hL = rng.uniform(0.2, 10.0, n)
    hR = rng.uniform(0.2, 10.0, n)
    qL = rng.uniform(-3, 3, n) * hL
    qR = rng.uniform(-3, 3, n) * hR
    tL = rng.uniform(-2, 2, n) * hL
    tR = rng.uniform(-2, 2, n) * hR
    cL = rng.uniform(0, 1, n) * hL
    cR = rng.uniform(0, 1, n) * hR
    HL = rng.uniform(-1, 1, n)
    HR = rng.uniform(-1, 1, n)
    return [(np.array([hL[i], qL[i], tL[i], cL[i], HL[i]]),
             np.array([hR[i], qR[i], tR[i], cR[i], HR[i]])) for i in range(n)]


def test_roe1_matches_library_eigendecomposition():
    rng = np.random.default_rng(11)
    worst = 0.0
    for L, R in _random_states1(rng, 4000):
        phi, sp = oracle.roe1_edge(L, R, G)
        u, h = _roe_avg(L[0], L[1], R[0], R[1])
        A = np.array([[0.0, 1.0], [G * h - u * u, 2.0 * u]])
        P, lam = _pminus(A)
        F = lambda s: np.array([s[1], s[1] ** 2 / s[0] + 0.5 * G * s[0] ** 2])
        X = F(R) - F(L) - np.array([0.0, G * h]) * (R[4] - L[4])
        ref = F(L) + P @ X
        scale = np.abs(F(L)).max() + np.abs(X).max()
        worst = max(worst, np.abs(phi[:2] - ref).max() / scale)
        assert sp == pytest.approx(np.abs(lam).max(), rel=1e-13)
        up = L if phi[0] > 0 else R
        assert phi[2] == pytest.approx(phi[0] * up[2] / up[0], rel=1e-13, abs=1e-300)
        assert phi[3] == pytest.approx(phi[0] * up[3] / up[0], rel=1e-13, abs=1e-300)
    assert worst < 1e-12


def test_roe1_supersonic_is_upwind():
    # all waves to the right: the flux is the left physical flux, exactly
    L = np.array([1.0, 8.0, 0.3, 0.5, 0.2])
    R = np.array([1.3, 9.0, -0.1, 0.1, -0.4])
    phi, _ = oracle.roe1_edge(L, R, G)
    assert phi[0] == L[1]
    assert phi[1] == L[1] ** 2 / L[0] + 0.5 * G * L[0] ** 2
    # all waves to the left: flux = F(W_R) - S dH
    L2 = _flip(R, [1, 2])
    R2 = _flip(L, [1, 2])
    phi2, _ = oracle.roe1_edge(L2, R2, G)
    h = 0.5 * (L2[0] + R2[0])
    F1R = R2[1] ** 2 / R2[0] + 0.5 * G * R2[0] ** 2
    assert phi2[0] == pytest.approx(R2[1], rel=1e-14)
    assert phi2[1] == pytest.approx(F1R - G * h * (R2[4] - L2[4]), rel=1e-14)


def test_roe1_consistency():
    # equal states on a flat bed: the numerical flux is the physical flux
    s = np.array([2.0, 1.5, -0.7, 0.4, 0.3])
    phi, sp = oracle.roe1_edge(s, s, G)
    assert phi[0] == s[1]
    assert phi[1] == pytest.approx(s[1] ** 2 / s[0] + 0.5 * G * s[0] ** 2, rel=1e-15)
    assert phi[2] == pytest.approx(s[1] * s[2] / s[0], rel=1e-15)
    assert sp == pytest.approx(abs(s[1] / s[0]) + math.sqrt(G * s[0]), rel=1e-15)


def test_roe1_still_water_is_balanced():
    # lake at rest: h + z equal, no velocity -> only the hydrostatic flux
    rng = np.random.default_rng(5)
    for _ in range(200):
        zL, zR = rng.uniform(-2, 2, 2)
        L = np.array([5.0 - zL, 0.0, 0.0, 0.0, -zL])
        R = np.array([5.0 - zR, 0.0, 0.0, 0.0, -zR])
        phi, _ = oracle.roe1_edge(L, R, G)
        assert abs(phi[0]) < 1e-13
        assert phi[1] == pytest.approx(0.5 * G * L[0] ** 2, rel=1e-14)


def test_roe1_wall_is_the_mirror_problem():
    rng = np.random.default_rng(3)
    for _ in range(200):
        h = rng.uniform(0.1, 10)
        q = rng.uniform(-5, 5) * h
        L = np.array([h, q, rng.uniform(-1, 1), rng.uniform(0, h), 0.2])
        wall, spw = oracle.roe1_wall(L, G)
        mirror, spm = oracle.roe1_edge(L, _flip(L, [1]), G)
        assert wall[0] == 0.0 and wall[2] == 0.0 and wall[3] == 0.0
        assert abs(mirror[0]) <= 1e-14 * abs(q) + 1e-300
        assert wall[1] == pytest.approx(mirror[1], rel=1e-14)
        assert spw == pytest.approx(spm, rel=1e-15)


def test_roe1_path_conservative_jump():
    # flux leaving i minus flux entering j = S_ij (H_j - H_i) in the normal
    # momentum row only; mass, transverse momentum and pollutant are
    # conserved (evaluated independently from both sides of the edge)
    rng = np.random.default_rng(7)
    for L, R in _random_states1(rng, 2000):
        phi_ij, _ = oracle.roe1_edge(L, R, G)
        phi_ji, _ = oracle.roe1_edge(_flip(R, [1, 2]), _flip(L, [1, 2]), G)
        into_j = np.array([-phi_ji[0], phi_ji[1], phi_ji[2], -phi_ji[3]])
        h = 0.5 * (L[0] + R[0])
        scale = abs(phi_ij).max() + 1.0
        assert abs(into_j[0] - phi_ij[0]) < 1e-13 * scale
        assert abs(into_j[2] - phi_ij[2]) < 1e-13 * scale
        assert abs(into_j[3] - phi_ij[3]) < 1e-13 * scale
        assert abs((into_j[1] - phi_ij[1]) - G * h * (R[4] - L[4])) < 1e-12 * scale


# --------------------------------------------------------------- two layers

def _A2(L, R, r):
    u1, h1 = _roe_avg(L[0], L[1], R[0], R[1])
    u2, h2 = _roe_avg(L[3], L[4], R[3], R[4])
    A = np.array([[0, 1, 0, 0],
                  [G * h1 - u1 * u1, 2 * u1, G * h1, 0],
                  [0, 0, 0, 1],
                  [r * G * h2, 0, G * h2 - u2 * u2, 2 * u2]], dtype=float)
    return A, h1, h2


def _random_states2(rng, n):
    out = []
    while len(out) < n:
        h1 = rng.uniform(0.5, 4.0, 2)
        h2 = rng.uniform(0.5, 4.0, 2)
        u1 = rng.uniform(-0.6, 0.6, 2)
        u2 = u1 + rng.uniform(-0.2, 0.2, 2)
        t = rng.uniform(-0.5, 0.5, 4)
        H = rng.uniform(-0.5, 0.5, 2)
        L = np.array([h1[0], u1[0] * h1[0], t[0], h2[0], u2[0] * h2[0], t[1], H[0]])
        R = np.array([h1[1], u1[1] * h1[1], t[2], h2[1], u2[1] * h2[1], t[3], H[1]])
        A, _, _ = _A2(L, R, 0.98)
        if np.all(np.abs(np.linalg.eigvals(A).imag) == 0.0):
            out.append((L, R))
    return out


def test_roe2_eigenvalues_match_library():
    rng = np.random.default_rng(21)
    for L, R in _random_states2(rng, 1500):
        _, sp, lam = oracle.roe2_edge(L, R, G, 0.98)
        A, _, _ = _A2(L, R, 0.98)
        ref = np.sort(np.linalg.eigvals(A).real)
        assert np.abs(lam - ref).max() < 1e-10 * np.abs(ref).max()
        assert sp == pytest.approx(np.abs(ref).max(), rel=1e-10)


def test_roe2_eigenvalues_closed_form_equal_velocities():
    # u1 = u2 = u: lambda = u +- sqrt(x), x the roots of
    # x^2 - (c1^2 + c2^2) x + (1 - r) c1^2 c2^2 = 0
    for (h1, h2, u, r) in [(2.5, 2.5, 0.0, 0.98), (1.0, 3.0, 0.4, 0.9), (2.0, 0.7, -0.3, 0.5)]:
        L = np.array([h1, u * h1, 0.0, h2, u * h2, 0.0, 0.0])
        _, _, lam = oracle.roe2_edge(L, L, G, r)
        a, b = G * h1, G * h2
        disc = math.sqrt((a + b) ** 2 - 4 * (1 - r) * a * b)
        xs = [(a + b + disc) / 2, (a + b - disc) / 2]
        ref = sorted([u - math.sqrt(xs[0]), u - math.sqrt(xs[1]),
                      u + math.sqrt(xs[1]), u + math.sqrt(xs[0])])
        assert np.allclose(lam, ref, rtol=0, atol=1e-12)
    # the rest state of the two-layer workload: external and internal speeds
    L = np.array([2.5, 0.0, 0.0, 2.5, 0.0, 0.0, 0.0])
    _, sp, lam = oracle.roe2_edge(L, L, G, 0.98)
    assert sp == pytest.approx(6.98595, abs=5e-6)
    assert lam[2] == pytest.approx(0.49648, abs=5e-6)


def test_roe2_flux_matches_library_eigendecomposition():
    rng = np.random.default_rng(22)
    worst = 0.0
    for L, R in _random_states2(rng, 1500):
        phi, _, _ = oracle.roe2_edge(L, R, G, 0.98)
        A, h1, h2 = _A2(L, R, 0.98)
        P, _ = _pminus(A)
        F = lambda s: np.array([s[1], s[1] ** 2 / s[0] + 0.5 * G * s[0] ** 2,
                                s[4], s[4] ** 2 / s[3] + 0.5 * G * s[3] ** 2])
        dh1, dh2, dH = R[0] - L[0], R[3] - L[3], R[6] - L[6]
        BdW = np.array([0.0, -G * h1 * dh2, 0.0, -0.98 * G * h2 * dh1])
        SdH = np.array([0.0, G * h1, 0.0, G * h2]) * dH
        X = F(R) - F(L) - BdW - SdH
        ref = F(L) + P @ X
        got = phi[[0, 1, 3, 4]]
        scale = np.abs(F(L)).max() + np.abs(X).max()
        worst = max(worst, np.abs(got - ref).max() / scale)
        up1 = L if phi[0] > 0 else R
        up2 = L if phi[3] > 0 else R
        assert phi[2] == pytest.approx(phi[0] * up1[2] / up1[0], rel=1e-13, abs=1e-300)
        assert phi[5] == pytest.approx(phi[3] * up2[5] / up2[3], rel=1e-13, abs=1e-300)
    assert worst < 1e-10


def test_roe2_total_momentum_identity():
    # Seen from both sides, layer masses are conserved and the momentum jumps
    # are the non-conservative products.  On a flat bed the density-weighted
    # sum rho1 q1 + rho2 q2 jumps by -r g d(h1 h2): the discrete form of the
    # two-layer system's total momentum balance, which holds only when r
    # multiplies the lower layer's coupling term.
    rng = np.random.default_rng(23)
    for L, R in _random_states2(rng, 800):
        for flat in (False, True):
            if flat:
                R = R.copy()
                R[6] = L[6]
            phi_ij, _, _ = oracle.roe2_edge(L, R, G, 0.98)
            phi_ji, _, _ = oracle.roe2_edge(_flip(R, [1, 2, 4, 5]), _flip(L, [1, 2, 4, 5]), G, 0.98)
            into_j = np.array([-phi_ji[0], phi_ji[1], phi_ji[2], -phi_ji[3], phi_ji[4], phi_ji[5]])
            scale = np.abs(phi_ij).max() + 1.0
            h1 = 0.5 * (L[0] + R[0]); h2 = 0.5 * (L[3] + R[3])
            dh1, dh2, dH = R[0] - L[0], R[3] - L[3], R[6] - L[6]
            assert abs(into_j[0] - phi_ij[0]) < 1e-11 * scale
            assert abs(into_j[3] - phi_ij[3]) < 1e-11 * scale
            j1 = into_j[1] - phi_ij[1]
            j2 = into_j[4] - phi_ij[4]
            assert abs(j1 - (-G * h1 * dh2 + G * h1 * dH)) < 1e-10 * scale
            assert abs(j2 - (-0.98 * G * h2 * dh1 + G * h2 * dH)) < 1e-10 * scale
            if flat:
                d12 = R[0] * R[3] - L[0] * L[3]
                assert abs(0.98 * j1 + j2 + 0.98 * G * d12) < 1e-10 * scale


def test_roe2_wall_zero_mass_flux():
    L = np.array([2.0, 0.7, 0.1, 3.0, -0.4, 0.2, 0.0])
    phi, sp = oracle.roe2_wall(L, G, 0.98)
    assert phi[0] == 0.0 and phi[2] == 0.0 and phi[3] == 0.0 and phi[5] == 0.0
    full, sp2, _ = oracle.roe2_edge(L, _flip(L, [1, 4]), G, 0.98)
    assert abs(full[0]) < 1e-12 and abs(full[3]) < 1e-12
    assert phi[1] == pytest.approx(full[1], rel=1e-13)
    assert phi[4] == pytest.approx(full[4], rel=1e-13)
    assert sp == sp2


def test_roe2_nonhyperbolic_is_reported():
    # a large velocity shear between the layers makes the internal roots complex
    L = np.array([2.0, 2.0 * 1.5, 0.0, 2.0, -2.0 * 1.5, 0.0, 0.0])
    with pytest.raises(oracle.OracleError) as e:
        oracle.roe2_edge(L, L, G, 0.98)
    assert e.value.code == 4


# ------------------------------------------- one layer, classical Roe variant

def _classical_matrix(L, R):
    """Roe matrix of (h, q_n, q_t, hc) at the Roe state, from its definition."""
    sL, sR = math.sqrt(L[0]), math.sqrt(R[0])
    avg = lambda a, b: (sL * a + sR * b) / (sL + sR)
    u = avg(L[1] / L[0], R[1] / R[0])
    v = avg(L[2] / L[0], R[2] / R[0])
    C = avg(L[3] / L[0], R[3] / R[0])
    h = 0.5 * (L[0] + R[0])
    A = np.array([[0.0, 1.0, 0.0, 0.0],
                  [G * h - u * u, 2.0 * u, 0.0, 0.0],
                  [-u * v, v, u, 0.0],
                  [-u * C, C, 0.0, u]])
    return A, h


def _F4(s):
    return np.array([s[1], s[1] ** 2 / s[0] + 0.5 * G * s[0] ** 2, s[1] * s[2] / s[0], s[1] * s[3] / s[0]])


def test_roe1c_matches_library_eigendecomposition():
    rng = np.random.default_rng(17)
    states = _random_states1(rng, 3000)
    # a zero Roe velocity (contact waves split half and half) and equal depths
    states.append((np.array([2.0, 1.0, 0.4, 0.3, 0.1]), np.array([2.0, -1.0, -0.2, 0.9, 0.0])))
    worst = 0.0
    for L, R in states:
        phi, sp = oracle.roe1c_edge(L, R, G)
        A, h = _classical_matrix(L, R)
        P, lam = _pminus(A)
        X = _F4(R) - _F4(L) - np.array([0.0, G * h, 0.0, 0.0]) * (R[4] - L[4])
        ref = _F4(L) + P @ X
        scale = np.abs(_F4(L)).max() + np.abs(X).max()
        worst = max(worst, np.abs(phi - ref).max() / scale)
        assert sp == pytest.approx(np.abs(lam).max(), rel=1e-13)
    assert worst < 1e-12


def test_roe1c_mass_and_normal_momentum_equal_ir_roe():
    # the 2x2 part (mass, normal momentum) is the same system in both schemes
    rng = np.random.default_rng(19)
    for L, R in _random_states1(rng, 500):
        a, _ = oracle.roe1_edge(L, R, G)
        b, _ = oracle.roe1c_edge(L, R, G)
        assert np.abs(a[:2] - b[:2]).max() <= 1e-14 * (np.abs(a[:2]).max() + 1.0)


def test_roe1c_consistency_and_constant_concentration():
    s = np.array([1.7, 0.8, -0.3, 0.6, 0.2])
    phi, _ = oracle.roe1c_edge(s, s, G)
    # F(W, W) = F(W) exactly (X = 0), with F_t = q (t / h), F_c = q (hc / h)
    Fs = np.array([s[1], s[1] * s[1] / s[0] + 0.5 * G * s[0] * s[0], s[1] * (s[2] / s[0]), s[1] * (s[3] / s[0])])
    assert np.array_equal(phi, Fs)
    L = np.array([1.2, 0.5, 0.1, 1.2, 0.0])               # hc = h: concentration 1
    R = np.array([0.7, -0.2, 0.3, 0.7, 0.3])
    phi, _ = oracle.roe1c_edge(L, R, G)
    assert phi[3] == phi[0]                               # pollutant flux = mass flux, bitwise


def test_roe1c_contact_wave_upwinds_by_roe_velocity():
    # mass flux into R (> 0) but a Roe velocity < 0: the IR-Roe scheme takes
    # the transverse velocity from L, the contact wave of the classical one
    # from R -- the two transverse fluxes must differ and the classical one
    # must follow the library decomposition (checked above); here its
    # closed form: Phi_t = F_t(L) + v P0 + [u < 0] (X_t - v X_0)
    L = np.array([3.0, 0.2, 1.5, 0.0, 0.0])
    R = np.array([1.0, -0.9, -0.7, 0.0, 0.0])
    ir, _ = oracle.roe1_edge(L, R, G)
    cl, _ = oracle.roe1c_edge(L, R, G)
    A, h = _classical_matrix(L, R)
    u, v = A[2, 2], A[2, 1]
    assert u < 0.0 and ir[0] > 0.0
    X = _F4(R) - _F4(L)
    P0 = cl[0] - L[1]
    ref = L[1] * L[2] / L[0] + v * P0 + (X[2] - v * X[0])
    assert cl[2] == pytest.approx(ref, rel=1e-13)
    assert abs(cl[2] - ir[2]) > 1e-3


def test_roe1c_test_matrix_has_the_roe_property():
    # the matrix the classical pins compare against is itself pinned: a Roe
    # matrix maps the jump of the state to the jump of the flux exactly
    # (normal row: up to the hydrostatic term g hbar dh, which is exact too)
    rng = np.random.default_rng(23)
    for L, R in _random_states1(rng, 500):
        A, h = _classical_matrix(L, R)
        dW = (R - L)[:4]
        dF = _F4(R) - _F4(L)
        assert np.abs(A @ dW - dF).max() <= 1e-12 * (np.abs(dF).max() + 1.0)


# ------------------------------------------------------- classical, 2 layers

def _F6(s):
    """flux of (h1, q1n, q1t, h2, q2n, q2t) along the normal (no coupling)"""
    return np.array([s[1], s[1] ** 2 / s[0] + 0.5 * G * s[0] ** 2, s[1] * s[2] / s[0],
                     s[4], s[4] ** 2 / s[3] + 0.5 * G * s[3] ** 2, s[4] * s[5] / s[3]])


def _A6(L, R, r):
    """Full two-layer Roe matrix J6 - B6 on (h1, q1n, q1t, h2, q2n, q2t) and
    the parts of the path-conservative jump: returns (A6, B6, S6)."""
    rows = {}
    for k, o in enumerate((0, 3)):
        sL, sR = math.sqrt(L[o]), math.sqrt(R[o])
        avg = lambda a, b: (sL * a + sR * b) / (sL + sR)
        rows[k] = (avg(L[o + 1] / L[o], R[o + 1] / R[o]), avg(L[o + 2] / L[o], R[o + 2] / R[o]),
                   0.5 * (L[o] + R[o]))
    (u1, v1, h1), (u2, v2, h2) = rows[0], rows[1]
    J = np.zeros((6, 6))
    J[0, 1] = 1.0
    J[1, 0], J[1, 1] = G * h1 - u1 * u1, 2 * u1
    J[2, 0], J[2, 1], J[2, 2] = -u1 * v1, v1, u1
    J[3, 4] = 1.0
    J[4, 3], J[4, 4] = G * h2 - u2 * u2, 2 * u2
    J[5, 3], J[5, 4], J[5, 5] = -u2 * v2, v2, u2
    B = np.zeros((6, 6))
    B[1, 3] = -G * h1
    B[4, 0] = -r * G * h2
    S = np.array([0.0, G * h1, 0.0, 0.0, G * h2, 0.0])
    return J - B, J, B, S


def _distinct6(rng, n):
    # states whose six eigenvalues are real and apart (a library
    # eigen-decomposition is well conditioned there)
    out = []
    for L, R in _random_states2(rng, 3 * n):
        A, _, _, _ = _A6(L, R, 0.98)
        lam = np.linalg.eigvals(A)
        d = np.abs(lam[:, None] - lam[None, :]) + np.eye(6)
        if np.abs(lam.imag).max() == 0.0 and d.min() > 0.05:
            out.append((L, R))
        if len(out) == n:
            break
    return out


def test_roe2c_test_matrix_has_the_roe_property():
    rng = np.random.default_rng(31)
    for L, R in _random_states2(rng, 300):
        _, J, _, _ = _A6(L, R, 0.98)
        dW = (R - L)[:6]
        dF = _F6(R) - _F6(L)
        assert np.abs(J @ dW - dF).max() <= 1e-12 * (np.abs(dF).max() + 1.0)


def test_roe2c_matches_library_eigendecomposition():
    rng = np.random.default_rng(32)
    states = _distinct6(rng, 800)
    assert len(states) >= 400
    worst = 0.0
    for L, R in states:
        phi, sp, _ = oracle.roe2c_edge(L, R, G, 0.98)
        A, _, B, S = _A6(L, R, 0.98)
        P, lam = _pminus(A)
        X = _F6(R) - _F6(L) - B @ (R - L)[:6] - S * (R[6] - L[6])
        ref = _F6(L) + P @ X
        scale = np.abs(_F6(L)).max() + np.abs(X).max()
        worst = max(worst, np.abs(phi - ref).max() / scale)
        assert sp == pytest.approx(np.abs(lam).max(), rel=1e-10)
    assert worst < 1e-10


def test_roe2c_normal_rows_and_speed_equal_ir_roe():
    # the normal system (h_k, q_kn) does not see the transverse momenta
    rng = np.random.default_rng(33)
    for L, R in _random_states2(rng, 500):
        a, sa, la = oracle.roe2_edge(L, R, G, 0.98)
        b, sb, lb = oracle.roe2c_edge(L, R, G, 0.98)
        n = [0, 1, 3, 4]
        assert np.abs(a[n] - b[n]).max() <= 1e-12 * (np.abs(a[n]).max() + 1.0)
        assert sa == sb and np.array_equal(la, lb)


def test_roe2c_uniform_transverse_velocity_equals_ir_roe():
    # with one transverse velocity per layer on both sides, the contact waves
    # carry nothing and both schemes move q_t with the mass flux
    rng = np.random.default_rng(34)
    for L, R in _random_states2(rng, 300):
        V1, V2 = rng.uniform(-1, 1, 2)
        L, R = L.copy(), R.copy()
        for s in (L, R):
            s[2], s[5] = V1 * s[0], V2 * s[3]
        a, _, _ = oracle.roe2_edge(L, R, G, 0.98)
        b, _, _ = oracle.roe2c_edge(L, R, G, 0.98)
        assert np.abs(a - b).max() <= 1e-11 * (np.abs(a).max() + 1.0)


def test_roe2c_consistency_and_pure_shear():
    s = np.array([1.4, 0.3, -0.2, 2.1, -0.1, 0.5, 0.2])
    phi, _, _ = oracle.roe2c_edge(s, s, G, 0.9)
    assert np.abs(phi - _F6(s)).max() <= 1e-14 * np.abs(_F6(s)).max()
    # same depths and normal discharges, flat bed, only q_t jumps: the
    # acoustic and internal waves carry nothing, each contact wave takes its
    # transverse flux from the upwind side of its own layer's velocity
    L = np.array([1.0, 0.4, 0.7, 2.0, -0.6, -0.3, 0.0])
    R = np.array([1.0, 0.4, -0.5, 2.0, -0.6, 0.9, 0.0])
    phi, _, _ = oracle.roe2c_edge(L, R, G, 0.98)
    FL, FR = _F6(L), _F6(R)
    assert np.abs(phi[[0, 1, 3, 4]] - FL[[0, 1, 3, 4]]).max() <= 1e-14 * np.abs(FL).max()
    assert phi[2] == pytest.approx(FL[2], rel=1e-14)      # u1 > 0: from L
    assert phi[5] == pytest.approx(FR[5], rel=1e-14)      # u2 < 0: from R


# ------------------------------------------------ Harten-Hyman entropy fix

def _subcritical_small_jumps(rng, n):
    # every state near the others and well below critical speed: no wave
    # can change the sign of its characteristic speed
    out = []
    for _ in range(n):
        h = rng.uniform(0.5, 5.0)
        hL, hR = h * rng.uniform(0.85, 1.15, 2)
        c = math.sqrt(G * h)
        uL, uR = rng.uniform(-0.3, 0.3, 2) * c
        out.append((np.array([hL, uL * hL, rng.uniform(-1, 1), 0.3 * hL, rng.uniform(-0.2, 0.2)]),
                    np.array([hR, uR * hR, rng.uniform(-1, 1), 0.6 * hR, rng.uniform(-0.2, 0.2)])))
    return out


def _transonic_dam_breaks(rng, n):
    # deep side at rest or slowly moving, shallow side much shallower: the
    # left rarefaction of the Riemann problem straddles the edge
    out = []
    for _ in range(n):
        hL = rng.uniform(1.0, 4.0)
        hR = hL * rng.uniform(0.01, 0.08)
        cL = math.sqrt(G * hL)
        L = np.array([hL, rng.uniform(0.0, 0.3) * cL * hL, rng.uniform(-1, 1), 0.5 * hL, rng.uniform(-0.05, 0.05)])
        R = np.array([hR, rng.uniform(0.0, 0.3) * cL * hR, rng.uniform(-1, 1), 0.2 * hR, rng.uniform(-0.05, 0.05)])
        out.append((L, R))
    return out


def test_entropy_fix_is_inactive_without_transonic_waves():
    rng = np.random.default_rng(41)
    for L, R in _subcritical_small_jumps(rng, 1000):
        a, sa = oracle.roe1_edge(L, R, G)
        b, sb = oracle.roe1_edge_fix(L, R, G)
        assert np.array_equal(a, b) and sa == sb
    # supercritical flow with moderate jumps: every speed has the sign of u
    for L, R in _subcritical_small_jumps(rng, 500):
        sg = rng.choice([-1.0, 1.0])
        for st in (L, R):
            st[1] = sg * rng.uniform(2.5, 3.5) * math.sqrt(G * st[0]) * st[0]
        a, _ = oracle.roe1_edge(L, R, G)
        b, _ = oracle.roe1_edge_fix(L, R, G)
        assert np.array_equal(a, b)
    # a lake at rest over a step
    L = np.array([2.0, 0.0, 0.0, 0.0, -0.3])
    R = np.array([1.7, 0.0, 0.0, 0.0, 0.0])
    assert np.array_equal(oracle.roe1_edge(L, R, G)[0], oracle.roe1_edge_fix(L, R, G)[0])


def test_entropy_fix_acts_on_transonic_rarefactions_and_stays_conservative():
    # the fix changes the flux, and seen from both sides of the edge mass,
    # transverse momentum and pollutant are still conserved and the normal
    # momentum jump is still S dH (a wave is split, its total flux jump kept)
    rng = np.random.default_rng(42)
    changed = 0
    for L, R in _transonic_dam_breaks(rng, 1000):
        phi_ij, _ = oracle.roe1_edge_fix(L, R, G)
        plain, _ = oracle.roe1_edge(L, R, G)
        changed += not np.array_equal(phi_ij, plain)
        phi_ji, _ = oracle.roe1_edge_fix(_flip(R, [1, 2]), _flip(L, [1, 2]), G)
        into_j = np.array([-phi_ji[0], phi_ji[1], phi_ji[2], -phi_ji[3]])
        h = 0.5 * (L[0] + R[0])
        scale = abs(phi_ij).max() + 1.0
        assert abs(into_j[0] - phi_ij[0]) < 1e-13 * scale
        assert abs(into_j[2] - phi_ij[2]) < 1e-13 * scale
        assert abs(into_j[3] - phi_ij[3]) < 1e-13 * scale
        assert abs((into_j[1] - phi_ij[1]) - G * h * (R[4] - L[4])) < 1e-12 * scale
    assert changed > 800   # most of these straddle the edge


def test_entropy_fix_of_the_classical_flux():
    # the fix acts on the acoustic waves only: inactive where no wave is
    # transonic; on transonic states its change of the classical flux is the
    # IR-Roe flux's change in mass and normal momentum, carried along the
    # acoustic eigenvectors (1, lam, vbar, Cbar) in the other two rows, and
    # the two sides of an edge still conserve mass, transverse momentum and
    # pollutant
    rng = np.random.default_rng(43)
    for L, R in _subcritical_small_jumps(rng, 300):
        assert np.array_equal(oracle.roe1c_edge(L, R, G)[0], oracle.roe1c_edge_fix(L, R, G)[0])
    for L, R in _transonic_dam_breaks(rng, 300):
        d_ir = oracle.roe1_edge_fix(L, R, G)[0] - oracle.roe1_edge(L, R, G)[0]
        d_cl = oracle.roe1c_edge_fix(L, R, G)[0] - oracle.roe1c_edge(L, R, G)[0]
        A, _ = _classical_matrix(L, R)
        vbar, Cbar = A[2, 1], A[3, 1]
        scale = abs(d_ir[:2]).max() + 1e-300
        assert abs(d_cl[0] - d_ir[0]) <= 1e-12 * scale and abs(d_cl[1] - d_ir[1]) <= 1e-12 * scale
        assert abs(d_cl[2] - vbar * d_cl[0]) <= 1e-12 * scale * (abs(vbar) + 1)
        assert abs(d_cl[3] - Cbar * d_cl[0]) <= 1e-12 * scale * (abs(Cbar) + 1)
        phi_ij, _ = oracle.roe1c_edge_fix(L, R, G)
        phi_ji, _ = oracle.roe1c_edge_fix(_flip(R, [1, 2]), _flip(L, [1, 2]), G)
        into_j = np.array([-phi_ji[0], phi_ji[1], phi_ji[2], -phi_ji[3]])
        s = abs(phi_ij).max() + 1.0
        assert abs(into_j[0] - phi_ij[0]) < 1e-13 * s
        assert abs(into_j[2] - phi_ij[2]) < 1e-13 * s
        assert abs(into_j[3] - phi_ij[3]) < 1e-13 * s
