"""Planted mistakes in the oracle must be caught by its pins.

Each entry plants one plausible mistake in a copy of oracle/swe_oracle.c (a
dropped factor, a wrong sign, a wrong upwind side, a wrong index, r in the
wrong row, a switch ignored, ...).  The fast test below only checks that
every planted snippet still occurs in the oracle, so that the list follows
the source.  The sweep itself -- build each broken copy and run the pin
tests (tests/test_oracle_flux.py, tests/test_oracle_invariants.py) against
it, expecting a failure -- takes a few minutes and runs when
SWE_ORACLE_MUTANTS=1 is set.  It plants mistakes in the oracle only, on the
CPU; the GPU path is not involved.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "..")
SRC = os.path.join(ROOT, "oracle", "swe_oracle.c")

# (name, exact text, replacement, occurrences)
MUTANTS = [
    # one layer, IR-Roe
    ("source sign", "double X1 = FR1 - FL1 - g * hbar * (HR - HL);",
     "double X1 = FR1 - FL1 + g * hbar * (HR - HL);", 1),
    ("source depth", "double X1 = FR1 - FL1 - g * hbar * (HR - HL);",
     "double X1 = FR1 - FL1 - g * hL * (HR - HL);", 1),
    ("sgn weight", "double w1 = 0.5 * (1.0 - sgn(lam1));", "double w1 = (1.0 - sgn(lam1));", 1),
    ("transverse upwind side", "double ustar = (f0 > 0.0) ? tL / hL : tR / hR;",
     "double ustar = (f0 > 0.0) ? tR / hR : tL / hL;", 1),
    ("pollutant upwind side", "double cstar = (f0 > 0.0) ? cL / hL : cR / hR;",
     "double cstar = (f0 < 0.0) ? cL / hL : cR / hR;", 1),
    ("wall term sign", "phi[1] = q * q / h + 0.5 * g * h * h + c * q;",
     "phi[1] = q * q / h + 0.5 * g * h * h - c * q;", 1),
    ("Roe average", "double ubar = (sL * uL + sR * uR) / (sL + sR);", "double ubar = 0.5 * (uL + uR);", 2),
    # geometry and time step
    ("triangle back-rotation", "a[1] += C->len[k] * (ex * phi[1] - ey * phi[2]);",
     "a[1] += C->len[k] * (ex * phi[1] + ey * phi[2]);", 1),
    ("grid back-rotation", "a[2] += len[sd] * (ey[sd] * phi[1] + ex[sd] * phi[2]);",
     "a[2] += len[sd] * (ey[sd] * phi[1] - ex[sd] * phi[2]);", 1),
    ("CFL factor", "dti[k] = 2.0 * cfl * area / S;", "dti[k] = cfl * area / S;", 1),
    ("triangle normal", "cells[t].ey[k] = -ddx / len;", "cells[t].ey[k] = ddx / len;", 1),
    ("periodic wrap", "if (periodic_x) ni = (ni + nx) % nx; else wall = 1;",
     "if (periodic_x) ni = (ni + nx - 1) % nx; else wall = 1;", 1),
    # two layers
    ("r in the upper layer", "                      {0.0, 0.0, -g * h1, 0.0},",
     "                      {0.0, 0.0, -r * g * h1, 0.0},", 1),
    ("r dropped", "                      {-r * g * h2, 0.0, 0.0, 0.0}};",
     "                      {-g * h2, 0.0, 0.0, 0.0}};", 1),
    ("two-layer source depth", "double S[4] = {0.0, g * h1, 0.0, g * h2};",
     "double S[4] = {0.0, g * h1L, 0.0, g * h2};", 1),
    ("two-layer upwind side", "double u2s = (f[2] > 0.0) ? t2L / h2L : t2R / h2R;",
     "double u2s = (f[2] > 0.0) ? t2R / h2R : t2L / h2L;", 1),
    # classical Roe, one layer
    ("classical transverse average", "double vbar = (sL * vL + sR * vR) / (sL + sR);",
     "double vbar = 0.5 * (vL + vR);", 1),
    ("classical contact strength", "al[1] = X[2] - vbar * X[0];", "al[1] = X[2] + vbar * X[0];", 1),
    ("classical eigenvector rows", "{{1.0, lam[0], vbar, Cbar},", "{{1.0, lam[0], Cbar, vbar},", 1),
    ("classical contact speed", "double lam[4] = {ubar - c, ubar, ubar, ubar + c};",
     "double lam[4] = {ubar - c, 0.0, ubar, ubar + c};", 1),
    ("classical switch ignored", "st = classical ? roe1_classical(Lst, Rst, g, fix, phi, &sp)",
     "st = 0 ? roe1_classical(Lst, Rst, g, fix, phi, &sp)", 2),
    # classical Roe, two layers
    ("classical 6x6 average", "double v1 = (s1L * (t1L / h1L) + s1R * (t1R / h1R)) / (s1L + s1R);",
     "double v1 = 0.5 * (t1L / h1L + t1R / h1R);", 1),
    ("classical 6x6 row sign", "{-u1 * v1, v1, u1, 0.0, 0.0, 0.0},", "{u1 * v1, v1, u1, 0.0, 0.0, 0.0},", 1),
    ("classical 6x6 contact speed", "mu[5] = u2;", "mu[5] = u1;", 1),
    ("classical 6x6 eigenvector completion", "K[t][k] = sum / (ev[k] - A[t][t]);",
     "K[t][k] = sum / (A[t][t] - ev[k]);", 1),
    ("classical 6x6 left flux", "q2L, q2L * q2L / h2L + 0.5 * g * h2L * h2L, q2L * t2L / h2L};",
     "q2L, q2L * q2L / h2L + 0.5 * g * h2L * h2L, q2L * t2R / h2L};", 1),
    ("classical 6x6 coupling", "B[4][0] = -r * g * h2;", "B[4][0] = -g * h2;", 1),
    ("classical 6x6 switch ignored", "st = classical ? or_roe2c_edge(Lst, Rst, g, r, phi, &sp, NULL)",
     "st = 0 ? or_roe2c_edge(Lst, Rst, g, r, phi, &sp, NULL)", 1),
    # Harten-Hyman entropy fix
    ("fix: wave strength sign", "double b1 = (lam2 * dh - dq) / (lam2 - lam1);",
     "double b1 = (dq - lam2 * dh) / (lam2 - lam1);", 1),
    ("fix: middle state", "double hs = hL + b1, qs = qL + b1 * lam1;", "double hs = hL + b2, qs = qL + b2 * lam1;", 1),
    ("fix: split fraction", "double lb = l1L * (l1R - lam1) / (l1R - l1L);",
     "double lb = l1L * (lam1 - l1L) / (l1R - l1L);", 1),
    ("fix: split speed", "double lb = l1L * (l1R - lam1) / (l1R - l1L);",
     "double lb = l1R * (l1R - lam1) / (l1R - l1L);", 1),
    ("fix: Roe part not removed", "double corr = lb - fmin(lam1, 0.0);", "double corr = lb - lam1;", 1),
    ("fix: second wave speed", "double lb = l2L * (l2R - lam2) / (l2R - l2L);",
     "double lb = l2R * (l2R - lam2) / (l2R - l2L);", 1),
    ("fix: momentum row", "*P1 += corr * b1 * lam1;", "*P1 += corr * b1 * lam2;", 1),
    ("fix: left speed", "double l1L = uL - sqrt(g * hL), l1R = us - cs;",
     "double l1L = uL - sqrt(g * hs), l1R = us - cs;", 1),
    ("fix: switch ignored", "if (fix) hh_fix(L, R, g, lam1, lam2, &P0, &P1);",
     "if (0) hh_fix(L, R, g, lam1, lam2, &P0, &P1);", 1),
    ("fix: transonic test", "if (l1L < 0.0 && l1R > 0.0) {", "if (l1L < 0.0 || l1R > 0.0) {", 1),
    ("classical fix: transverse row", "        phi[2] += vbar * d0;", "        phi[2] += Cbar * d0;", 1),
    ("classical fix: switch ignored", "    if (fix) { /* the fix's change of the acoustic waves, along r1 and r4 */",
     "    if (0) { /* the fix's change of the acoustic waves, along r1 and r4 */", 1),
]


def test_every_planted_snippet_is_in_the_oracle():
    src = open(SRC).read()
    for name, old, new, n in MUTANTS:
        assert src.count(old) == n, name
        assert old != new, name


@pytest.mark.skipif(os.environ.get("SWE_ORACLE_MUTANTS") != "1",
                    reason="the planted-mistake sweep takes minutes; set SWE_ORACLE_MUTANTS=1")
def test_planted_mistakes_are_caught():
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    src = open(SRC).read()
    missed = []
    with tempfile.TemporaryDirectory() as tmp:
        for i, (name, old, new, n) in enumerate(MUTANTS):
            c = os.path.join(tmp, f"m{i}.c")
            so = os.path.join(tmp, f"m{i}.so")
            open(c, "w").write(src.replace(old, new))
            obuild.build(src=c, lib=so)
            env = dict(os.environ, SWE_ORACLE_LIB=so)
            env.pop("SWE_ORACLE_MUTANTS", None)
            r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                                os.path.join(ROOT, "tests", "test_oracle_flux.py"),
                                os.path.join(ROOT, "tests", "test_oracle_invariants.py")],
                               env=env, capture_output=True, text=True, cwd=ROOT)
            print(name, "caught" if r.returncode else "MISSED", flush=True)
            if r.returncode == 0:
                missed.append(name)
    assert not missed, missed
