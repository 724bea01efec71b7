"""CPU oracle for the batched banded solvers -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it, and
it never imports the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one system at
a time, flat layout).  This module compiles it with gcc (``build()``) and
wraps it for numpy arrays.  All wrappers take and return FLAT arrays of shape
``(batch, n)`` (one system per row); use ``workloads.to_flat`` to convert the
interleaved GPU layout.  float32 inputs are promoted to float64 first, so the
oracle of an fp32 problem is the fp64 solve of the fp32-rounded inputs.

Functions and the passages they follow:
  penta_solve            -- cuPentBatch page, "Pentadiagonal solver":
                            factorisation steps 1-14, forward and back steps
  penta_factor           -- the same factorisation, returning the factors
  penta_cyclic_solve     -- cuPentBatch page, hyperdiffusion section: periodic
                            matrix and Navon's reduction, eqs. (10)-(12)
  hyperdiffusion         -- cuPentBatch page, eqs. (4)-(7) with the implicit
                            step (I + sigma D4) C^{n+1} = C^n, sigma = dt/dx^4
  hyperdiffusion_theta   -- cuPentBatch page, hyperdiffusion section: the
                            Crank-Nicolson step generalised to the theta family
  cahn_hilliard          -- cuPentBatch page, introduction: the Cahn-Hilliard
                            equation with the phase-separation term at the old
                            time level and the fourth-order term implicit
  thomas_solve           -- Hines page, section 4.1: Thomas algorithm for
                            tridiagonal systems (cuThomasBatch's method)
  hines_solve            -- Hines page, section 2, Algorithm 1
  hines_multi_solve      -- Algorithm 1 per neuron, one tree per neuron
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


# The CPU-baseline timing build: the same source with the flags of a tuned
# CPU build.  -march=native targets the host that compiles it, so it is built
# on the machine that runs the timing (build_timing), never shipped.
TIMING_CFLAGS = ["-O3", "-march=native", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                 "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liborc.so with gcc (plain -O2, no -march)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_timing(outdir: str) -> str:
    """Compile oracle.c with TIMING_CFLAGS into outdir/liborc_timing.so."""
    out = os.path.join(outdir, "liborc_timing.so")
    subprocess.check_call(["gcc", *TIMING_CFLAGS, _SRC, "-o", out, "-lm"])
    return out


def use_library(path: str) -> None:
    """Route every wrapper below through the build at `path` (the timing
    build, or the checker's liborc.so again); the thread count set by
    set_threads applies to the build loaded when it is called."""
    global _LIB_ACTIVE, _lib
    with _lock:
        if _LIB_ACTIVE != path:
            _lib = None
        _LIB_ACTIVE = path


_LIB_ACTIVE = _LIB


_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_ACTIVE == _LIB and (not os.path.exists(_LIB) or
                                        os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
            lib = ctypes.CDLL(_LIB_ACTIVE)
            lib.orc_set_threads.argtypes = [ctypes.c_int]
            lib.orc_set_threads.restype = ctypes.c_int
            lib.orc_penta_factor.argtypes = [_i64] + [_D] * 9
            lib.orc_penta_factor.restype = ctypes.c_int
            lib.orc_penta_solve.argtypes = [_i64] + [_D] * 7
            lib.orc_penta_solve.restype = ctypes.c_int
            lib.orc_penta_cyclic_solve.argtypes = [_i64] + [_D] * 7
            lib.orc_penta_cyclic_solve.restype = ctypes.c_int
            lib.orc_penta_cyclic_setup.argtypes = [_i64] + [_D] * 6
            lib.orc_penta_cyclic_setup.restype = ctypes.c_int
            lib.orc_penta_solve_batch.argtypes = [_i64, _i64, _i64] + [_D] * 6 + [_I32]
            lib.orc_penta_solve_batch.restype = None
            lib.orc_penta_cyclic_solve_batch.argtypes = [_i64, _i64, _i64] + [_D] * 6 + [_I32]
            lib.orc_penta_cyclic_solve_batch.restype = None
            lib.orc_hyperdiffusion.argtypes = [_i64, _i64, ctypes.c_double, ctypes.c_double,
                                               _D, _D, _i64]
            lib.orc_hyperdiffusion.restype = ctypes.c_int
            lib.orc_hyperdiffusion_theta.argtypes = [_i64, _i64, ctypes.c_double, ctypes.c_double,
                                                     ctypes.c_double, _D, _i64]
            lib.orc_hyperdiffusion_theta.restype = ctypes.c_int
            lib.orc_cahn_hilliard.argtypes = [_i64, _i64, ctypes.c_double, ctypes.c_double,
                                              ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                              _D, _i64]
            lib.orc_cahn_hilliard.restype = ctypes.c_int
            lib.orc_thomas_solve_batch.argtypes = [_i64, _i64, _D, _D, _D, _D, _I32]
            lib.orc_thomas_solve_batch.restype = None
            lib.orc_hines_solve.argtypes = [_i64, _I32, _D, _D, _D, _D]
            lib.orc_hines_solve.restype = ctypes.c_int
            lib.orc_hines_solve_batch.argtypes = [_i64, _i64, _I32, _D, _D, _D, _D, _I32]
            lib.orc_hines_solve_batch.restype = None
            lib.orc_hines_multi_batch.argtypes = [_i64, _I64, _I32, _D, _D, _D, _D, _I32]
            lib.orc_hines_multi_batch.restype = None
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: np.ndarray, t=_D):
    return x.ctypes.data_as(t)


def set_threads(k: int = 0) -> int:
    """Set (k > 0) and return the OpenMP thread count the batch drivers use."""
    return int(_load().orc_set_threads(int(k)))


def _batch2(x) -> np.ndarray:
    x = _f64(x)
    return x[None, :] if x.ndim == 1 else x


# ----------------------------------------------------------------------------
# Pentadiagonal
# ----------------------------------------------------------------------------

def penta_factor(a, b, c, d, e):
    """Factors (alpha, beta, gamma, delta) of ONE system and the info code."""
    a, b, c, d, e = (_f64(v) for v in (a, b, c, d, e))
    n = a.shape[0]
    if n < 4:
        raise ValueError("pentadiagonal solve needs n >= 4")
    out = [np.zeros(n) for _ in range(4)]
    info = _load().orc_penta_factor(n, *(_ptr(v) for v in (a, b, c, d, e)),
                                    *(_ptr(v) for v in out))
    return (*out, int(info))


def _diag_args(diags, n, batch):
    ds = [_f64(v) for v in diags]
    shared = ds[0].ndim == 1
    for v in ds:
        if shared and v.shape != (n,):
            raise ValueError("shared diagonals must have shape (n,)")
        if not shared and v.shape != (batch, n):
            raise ValueError("per-system diagonals must have shape (batch, n)")
    return ds, (0 if shared else n)


def penta_solve(a, b, c, d, e, f, cyclic: bool = False):
    """x = A^{-1} f for a batch (flat layout).

    Diagonals of shape (batch, n) (per system) or (n,) (shared by every
    system, factored once).  Returns (x, info) with x of shape (batch, n).
    """
    x = _batch2(f).copy()
    batch, n = x.shape
    if n < (6 if cyclic else 4):
        raise ValueError("n too small")
    ds, stride = _diag_args((a, b, c, d, e), n, batch)
    info = np.zeros(batch, dtype=np.int32)
    fn = _load().orc_penta_cyclic_solve_batch if cyclic else _load().orc_penta_solve_batch
    fn(n, batch, stride, *(_ptr(v) for v in ds), _ptr(x), _ptr(info, _I32))
    return x, info


def penta_cyclic_solve(a, b, c, d, e, f):
    return penta_solve(a, b, c, d, e, f, cyclic=True)


def penta_cyclic_setup(a, b, c, d, e):
    """Stored quantities of the periodic reduction for ONE matrix:
    (rows of G E^{-1} as a (2, n-2) array, the 2x2 inverse, info)."""
    a, b, c, d, e = (_f64(v) for v in (a, b, c, d, e))
    n = a.shape[0]
    out = np.zeros(2 * (n - 2) + 4)
    info = _load().orc_penta_cyclic_setup(n, *(_ptr(v) for v in (a, b, c, d, e)), _ptr(out))
    m = n - 2
    return out[:2 * m].reshape(2, m), out[2 * m:].reshape(2, 2), int(info)


def hyperdiffusion_diagonals(n: int, dt: float, dx: float):
    """The five diagonals of I + sigma*D4, sigma = dt/dx^4 (D4 = [1,-4,6,-4,1])."""
    sigma = dt / (dx * dx * dx * dx)
    one = np.ones(n)
    return (sigma * one, -4.0 * sigma * one, (1.0 + 6.0 * sigma) * one,
            -4.0 * sigma * one, sigma * one)


def hyperdiffusion(C0, dt: float, dx: float, nsteps: int, diagonals=None):
    """C^{nsteps} from C^0 (flat (batch, n)) by repeated implicit steps."""
    C = _batch2(C0).copy()
    batch, n = C.shape
    if n < 6:
        raise ValueError("periodic solve needs n >= 6")
    if diagonals is not None:
        dg = np.ascontiguousarray(np.stack([_f64(v) for v in diagonals]))
        dp = _ptr(dg)
    else:
        dg = None
        dp = None
    _load().orc_hyperdiffusion(n, batch, float(dt), float(dx), dp, _ptr(C), int(nsteps))
    return C


def hyperdiffusion_theta(C0, dt: float, dx: float, theta: float, nsteps: int):
    """C^{nsteps} from C^0 (flat (batch, n)) by theta-scheme steps
    (I + theta sigma D4) C' = (I - (1 - theta) sigma D4) C, sigma = dt/dx^4."""
    C = _batch2(C0).copy()
    batch, n = C.shape
    if n < 6:
        raise ValueError("periodic solve needs n >= 6")
    _load().orc_hyperdiffusion_theta(n, batch, float(dt), float(dx), float(theta), _ptr(C),
                                     int(nsteps))
    return C


def hyperdiffusion_theta_operators(n: int, dt: float, dx: float, theta: float):
    """Stencil entries (e2, e1, e0) of I - (1-theta) sigma D4 and diagonals
    (a, b, c, d, e) of I + theta sigma D4, rounded as the solver rounds them."""
    sigma = dt / (dx * dx * dx * dx)
    si, se = theta * sigma, (1.0 - theta) * sigma
    one = np.ones(n)
    return ((-se, 4.0 * se, 1.0 - 6.0 * se),
            (si * one, -4.0 * si * one, (1.0 + 6.0 * si) * one, -4.0 * si * one, si * one))


def cahn_hilliard(C0, dt: float, dx: float, gamma: float, mobility: float, theta: float,
                  nsteps: int):
    """C^{nsteps} from C^0 (flat (batch, n)) by semi-implicit Cahn-Hilliard
    steps (I + theta sigma D4) C' = (I - (1-theta) sigma D4) C + r D2 (C^3 - C),
    r = mobility dt / dx^2, sigma = gamma r / dx^2 (theta = 1: the linear
    fourth-order term fully implicit)."""
    C = _batch2(C0).copy()
    batch, n = C.shape
    if n < 6:
        raise ValueError("periodic solve needs n >= 6")
    _load().orc_cahn_hilliard(n, batch, float(dt), float(dx), float(gamma), float(mobility),
                              float(theta), _ptr(C), int(nsteps))
    return C


def cahn_hilliard_operators(n: int, dt: float, dx: float, gamma: float, mobility: float,
                            theta: float):
    """(e2, e1, e0), r and the implicit diagonals (a, b, c, d, e) of the
    Cahn-Hilliard step, rounded as the solver rounds them."""
    r = mobility * dt / (dx * dx)
    sigma = gamma * r / (dx * dx)
    si, se = theta * sigma, (1.0 - theta) * sigma
    one = np.ones(n)
    return ((-se, 4.0 * se, 1.0 - 6.0 * se), r,
            (si * one, -4.0 * si * one, (1.0 + 6.0 * si) * one, -4.0 * si * one, si * one))


# ----------------------------------------------------------------------------
# Hines
# ----------------------------------------------------------------------------

def thomas_solve(a, b, c, y):
    """Thomas algorithm for a batch of tridiagonal systems (flat layout).

    a (sub-diagonal, a[:, 0] ignored), b (diagonal), c (super-diagonal,
    c[:, -1] ignored), y (right-hand side): (batch, n) or (n,).
    Returns (u, info)."""
    u = _batch2(y).copy()
    batch, n = u.shape
    a, b, c = (_batch2(v) for v in (a, b, c))
    for v in (a, b, c):
        if v.shape != (batch, n):
            raise ValueError("a, b, c must match y")
    if n < 1:
        raise ValueError("n >= 1 needed")
    info = np.zeros(batch, dtype=np.int32)
    _load().orc_thomas_solve_batch(n, batch, _ptr(a), _ptr(b), _ptr(c), _ptr(u), _ptr(info, _I32))
    return u, info


def hines_solve(parent, u, l, d, rhs):
    """Algorithm 1 for a batch of neurons sharing one tree (flat layout).

    parent: (n,) int; u, l, d, rhs: (batch, n) or (n,).  Returns (V, info).
    d is not modified.
    """
    p = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    V = _batch2(rhs).copy()
    batch, n = V.shape
    u, l, d = (_batch2(v) for v in (u, l, d))
    for v in (u, l, d):
        if v.shape != (batch, n):
            raise ValueError("u, l, d must match rhs")
    if n > 1 and not np.all((p[1:] >= 0) & (p[1:] < np.arange(1, n))):
        raise ValueError("parent[i] must lie in [0, i)")
    info = np.zeros(batch, dtype=np.int32)
    _load().orc_hines_solve_batch(n, batch, _ptr(p, _I32), _ptr(u), _ptr(l), _ptr(d),
                                  _ptr(V), _ptr(info, _I32))
    return V, info


def hines_multi_solve(offsets, parent, u, l, d, rhs):
    """Algorithm 1 per neuron, each neuron with its own tree.

    offsets: (batch+1,) int64; parent, u, l, d, rhs: concatenated per neuron.
    Returns (V concatenated, info per neuron).
    """
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    p = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    V = _f64(rhs).copy()
    u, l, d = (_f64(v) for v in (u, l, d))
    batch = len(off) - 1
    info = np.zeros(batch, dtype=np.int32)
    _load().orc_hines_multi_batch(batch, _ptr(off, _I64), _ptr(p, _I32), _ptr(u), _ptr(l),
                                  _ptr(d), _ptr(V), _ptr(info, _I32))
    return V, info
