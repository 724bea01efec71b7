"""Writes the exact-arithmetic fixtures in this folder.

Run:  python tests/golden/make_golden.py
Calls only oracle.referee (exact rational Gaussian elimination).  The
systems are small integer matrices drawn from a fixed seed; their exact
solutions are stored as fraction strings.  Matrices follow the definitions
on the pages:
  penta  -- cuPentBatch page, "Pentadiagonal solver" (five diagonals a..e)
  cyclic -- cuPentBatch page, hyperdiffusion section (periodic wrap mod n)
  hines  -- Hines page, section 2 (A[i][i]=d_i, A[p_i][i]=u_i, A[i][p_i]=l_i)
  tri    -- Hines page, section 4.1 (row i: a_i, b_i, c_i at columns i-1, i, i+1)
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle.referee import solve_exact  # noqa: E402


def dense_penta(dg, cyclic):
    n = len(dg[2])
    A = [[0] * n for _ in range(n)]
    for i in range(n):
        for k, v in zip(range(-2, 3), dg):
            j = i + k
            if cyclic:
                A[i][j % n] += v[i]
            elif 0 <= j < n:
                A[i][j] = v[i]
    return A


def dense_hines(p, u, l, d):
    n = len(d)
    A = [[0] * n for _ in range(n)]
    for i in range(n):
        A[i][i] = d[i]
    for i in range(1, n):
        A[p[i]][i] = u[i]
        A[i][p[i]] = l[i]
    return A


def main():
    rng = np.random.default_rng(777)
    penta, cyclic, hines = [], [], []
    for n in (4, 5, 6, 7, 9, 12):
        for _ in range(3):
            dg = [[int(v) for v in rng.integers(-4, 5, n)] for _ in range(5)]
            for i in range(n):      # keep leading pivots away from zero
                dg[2][i] = int(rng.integers(10, 20)) * (1 if rng.random() < .5 else -1)
            if n >= 4:
                dg[0][0] = dg[0][1] = dg[1][0] = 0
                dg[3][n - 1] = dg[4][n - 2] = dg[4][n - 1] = 0
            f = [int(v) for v in rng.integers(-9, 10, n)]
            x = solve_exact(dense_penta(dg, False), f)
            penta.append({"n": n, "a": dg[0], "b": dg[1], "c": dg[2], "d": dg[3], "e": dg[4],
                          "f": f, "x": [str(v) for v in x]})
    for n in (6, 7, 8, 10, 13):
        for _ in range(3):
            dg = [[int(v) for v in rng.integers(-4, 5, n)] for _ in range(5)]
            for i in range(n):
                dg[2][i] = int(rng.integers(17, 30))
            f = [int(v) for v in rng.integers(-9, 10, n)]
            x = solve_exact(dense_penta(dg, True), f)
            cyclic.append({"n": n, "a": dg[0], "b": dg[1], "c": dg[2], "d": dg[3], "e": dg[4],
                           "f": f, "x": [str(v) for v in x]})
    for n in (1, 2, 3, 5, 8, 11):
        for _ in range(3):
            p = [-1] + [int(rng.integers(max(0, i - 3), i)) for i in range(1, n)]
            u = [0] + [int(v) for v in rng.integers(-5, 6, n - 1)]
            l = [0] + [int(v) for v in rng.integers(-5, 6, n - 1)]
            d = [int(v) * (1 if rng.random() < .5 else -1) for v in rng.integers(20, 40, n)]
            f = [int(v) for v in rng.integers(-9, 10, n)]
            x = solve_exact(dense_hines(p, u, l, d), f)
            hines.append({"n": n, "parent": p, "u": u, "l": l, "d": d, "f": f,
                          "x": [str(v) for v in x]})
    tri = []
    for n in (1, 2, 3, 4, 7, 10):
        for _ in range(3):
            a = [0] + [int(v) for v in rng.integers(-6, 7, n - 1)]
            c = [int(v) for v in rng.integers(-6, 7, n - 1)] + [0]
            b = [int(v) * (1 if rng.random() < .5 else -1) for v in rng.integers(13, 30, n)]
            f = [int(v) for v in rng.integers(-9, 10, n)]
            A = [[0] * n for _ in range(n)]
            for i in range(n):
                A[i][i] = b[i]
                if i > 0:
                    A[i][i - 1] = a[i]
                if i < n - 1:
                    A[i][i + 1] = c[i]
            x = solve_exact(A, f)
            tri.append({"n": n, "a": a, "b": b, "c": c, "f": f, "x": [str(v) for v in x]})
    hdr = ("Exact solutions (fractions) of small integer systems, written by "
           "tests/golden/make_golden.py with oracle.referee.solve_exact.")
    for name, cases, cite in (
            ("exact_penta.json", penta, "cuPentBatch page, section 'Pentadiagonal solver'"),
            ("exact_cyclic.json", cyclic, "cuPentBatch page, hyperdiffusion section, periodic matrix"),
            ("exact_hines.json", hines, "Hines page, section 2, Hines matrix"),
            ("exact_tri.json", tri, "Hines page, section 4.1, tridiagonal matrix")):
        with open(os.path.join(HERE, name), "w") as fh:
            json.dump({"about": hdr, "matrix": cite, "cases": cases}, fh, indent=0)
            fh.write("\n")


if __name__ == "__main__":
    main()
