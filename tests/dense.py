"""Dense matrices straight from their definitions on the pages (test helper).

penta_dense    -- the pentadiagonal matrix of the cuPentBatch page,
                  "Pentadiagonal solver": row i holds a_i, b_i, c_i, d_i, e_i
                  at columns i-2 .. i+2 (entries outside the matrix dropped).
cyclic_dense   -- the periodic matrix of the hyperdiffusion section: the same
                  five diagonals with column indices modulo n.
hines_dense    -- the Hines matrix of the Hines page, section 2:
                  A[i][i] = d_i, A[p_i][i] = u_i, A[i][p_i] = l_i.
"""
import numpy as np


def penta_dense(a, b, c, d, e):
    n = len(c)
    A = np.zeros((n, n))
    for i in range(n):
        for k, v in zip(range(-2, 3), (a, b, c, d, e)):
            j = i + k
            if 0 <= j < n:
                A[i, j] = v[i]
    return A


def cyclic_dense(a, b, c, d, e):
    n = len(c)
    A = np.zeros((n, n))
    for i in range(n):
        for k, v in zip(range(-2, 3), (a, b, c, d, e)):
            A[i, (i + k) % n] += v[i]
    return A


def hines_dense(parent, u, l, d):
    n = len(d)
    A = np.diag(np.asarray(d, dtype=float))
    for i in range(1, n):
        A[parent[i], i] = u[i]
        A[i, parent[i]] = l[i]
    return A


def relerr(x, y):
    """Per-system normwise relative error max_s |x_s - y_s| / |y_s| (rows = systems)."""
    x = np.atleast_2d(x); y = np.atleast_2d(y)
    return float(np.max(np.linalg.norm(x - y, axis=1) / np.linalg.norm(y, axis=1)))
