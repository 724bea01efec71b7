"""Referee for tiny systems: textbook dense Gaussian elimination.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

``solve_exact`` runs Gaussian elimination with partial pivoting in exact
rational arithmetic (``fractions.Fraction``), so on integer or rational input
its answer is the true x = A^{-1} f with no rounding at all.  It shares no
arithmetic with ``oracle.c`` (dense storage, row exchanges, exact numbers),
which is what makes it a pin for the banded elimination rather than a copy.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Sequence


def solve_exact(A: Sequence[Sequence], f: Sequence) -> list:
    """Exact x with A x = f.  A: n x n, entries int / Fraction / float
    (floats are taken at their exact binary value).  Raises on singular A."""
    n = len(A)
    M = [[Fraction(v) for v in row] + [Fraction(f[i])] for i, row in enumerate(A)]
    for k in range(n):
        piv = max(range(k, n), key=lambda r: abs(M[r][k]))
        if M[piv][k] == 0:
            raise ZeroDivisionError("singular matrix")
        M[k], M[piv] = M[piv], M[k]
        for r in range(k + 1, n):
            if M[r][k] != 0:
                m = M[r][k] / M[k][k]
                for c in range(k, n + 1):
                    M[r][c] -= m * M[k][c]
    x = [Fraction(0)] * n
    for i in range(n - 1, -1, -1):
        s = M[i][n] - sum(M[i][j] * x[j] for j in range(i + 1, n))
        x[i] = s / M[i][i]
    return x
