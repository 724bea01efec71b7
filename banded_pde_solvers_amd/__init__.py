"""Python binding of libbps -- batched banded solvers for MI355X (gfx950).

A thin ctypes layer over the C ABI in ``include/bps.h``: it marshals torch
tensors (device memory, current HIP stream) into plain pointers and sizes and
raises ``BpsError`` on a non-OK status.  Every step of every solve runs in the
HIP kernels of ``libbps.so``; there is no Python or CPU fallback, and calling
anything here without the built library raises ``BpsLibraryMissing``.

Array conventions (see bps.h):
  * interleaved arrays are 2-D tensors of shape (n, ld) in C order, element
    (row i, system s) at [i, s]; the first ``batch`` columns are used
    (batch defaults to ld);
  * shared diagonals (BPS_SHARED_COEF) are 1-D tensors of length n;
  * dtypes: torch.float64 (BPS_F64) or torch.float32 (BPS_F32).
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "BpsError", "BpsLibraryMissing", "BPS_F32", "BPS_F64", "BPS_CYCLIC", "BPS_SHARED_COEF",
    "library_path", "load_library", "version",
    "bps_penta_factor_bytes", "bps_penta_work_bytes",
    "penta_factor_batch", "penta_solve_batch", "penta_cyclic_solve_batch",
    "penta_factor_solve_batch",
    "hyperdiffusion_work_bytes", "hyperdiffusion_step", "hyperdiffusion_step_noalloc",
    "hyperdiffusion_factor", "hyperdiffusion_solve",
    "BPS_NOALLOC_SCRATCH_BYTES",
    "hyperdiffusion_theta_work_bytes", "hyperdiffusion_theta_step",
    "cahn_hilliard_work_bytes", "cahn_hilliard_step",
    "tri_work_bytes", "tri_solve_batch",
    "HinesPlan", "hines_plan_create", "hines_plan_destroy", "hines_pack", "hines_unpack",
    "hines_work_bytes", "hines_solve_batch", "BPS_HINES_AUTO", "BPS_HINES_LANES",
    "BPS_HINES_LEVELS", "BPS_HINES_SPLIT", "hines_plan_create_sched", "hines_plan_elems",
    "hines_plan_unknowns", "hines_plan_uses_levels", "hines_plan_split", "hines_split_schedule",
    "BPS_HINES_SEP", "hines_plan_uses_sep", "hines_sep_schedule", "hines_sep_multi_layout",
    "bps_version", "bps_init", "bps_status_str", "bps_last_error", "PentaDesc",
]

BPS_F32 = 1
BPS_F64 = 2
BPS_CYCLIC = 0x1
BPS_SHARED_COEF = 0x2
BPS_HINES_AUTO = 0
BPS_HINES_LANES = 1
BPS_HINES_LEVELS = 2
BPS_HINES_SPLIT = 3
BPS_HINES_SEP = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "libbps.so")
_lock = threading.Lock()
_lib = None


class BpsError(RuntimeError):
    """A libbps call returned a non-OK status."""

    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class BpsLibraryMissing(RuntimeError):
    """libbps.so has not been built (python -m banded_pde_solvers_amd.build)."""


class PentaDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("n", ctypes.c_int64), ("batch", ctypes.c_int64), ("ld", ctypes.c_int64)]


def library_path() -> str:
    return _LIBPATH


def load_library():
    """Load libbps.so and declare the C signatures (raises if it is missing)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIBPATH):
            raise BpsLibraryMissing(
                f"{_LIBPATH} not found: build it with 'python -m banded_pde_solvers_amd.build'")
        L = ctypes.CDLL(_LIBPATH)
        vp, i32p, i64, st = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int64, ctypes.c_int
        dp = ctypes.POINTER(PentaDesc)
        sig = {
            "bps_status_str": ([st], ctypes.c_char_p),
            "bps_last_error": ([], ctypes.c_char_p),
            "bps_version": ([], ctypes.c_int),
            "bps_init": ([], st),
            "bps_penta_factor_bytes": ([dp], ctypes.c_size_t),
            "penta_factor_batch": ([dp, vp, vp, vp, vp, vp, vp, vp, vp], st),
            "penta_solve_batch": ([dp, vp, vp, vp], st),
            "penta_cyclic_solve_batch": ([dp, vp, vp, vp], st),
            "bps_penta_work_bytes": ([dp], ctypes.c_size_t),
            "penta_factor_solve_batch": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp], st),
            "hyperdiffusion_work_bytes": ([st, i64, i64], ctypes.c_size_t),
            "hyperdiffusion_step": ([st, i64, i64, i64, ctypes.c_double, ctypes.c_double, vp, vp,
                                     i64, vp, vp], st),
            "hyperdiffusion_factor": ([st, i64, ctypes.c_double, ctypes.c_double, vp, vp, vp], st),
            "hyperdiffusion_solve": ([st, i64, i64, i64, ctypes.c_double, ctypes.c_double, vp, vp,
                                      i64, vp, vp], st),
            "hyperdiffusion_step_noalloc": ([st, i64, i64, i64, ctypes.c_double, ctypes.c_double,
                                             vp, vp, i64, vp], st),
            "hyperdiffusion_theta_work_bytes": ([st, i64, i64], ctypes.c_size_t),
            "hyperdiffusion_theta_step": ([st, i64, i64, i64, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, vp, i64, vp, vp], st),
            "cahn_hilliard_work_bytes": ([st, i64, i64], ctypes.c_size_t),
            "cahn_hilliard_step": ([st, i64, i64, i64, ctypes.c_double, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_double, ctypes.c_double, vp, i64,
                                    vp, vp], st),
            "tri_work_bytes": ([st, i64, i64], ctypes.c_size_t),
            "tri_solve_batch": ([st, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp], st),
            "hines_plan_create": ([ctypes.POINTER(vp), i64, i32p, i32p, st, i64], st),
            "hines_plan_create_sched": ([ctypes.POINTER(vp), i64, i32p, i32p, st, i64, st], st),
            "hines_plan_uses_levels": ([vp], st),
            "hines_plan_split": ([vp], i64),
            "hines_plan_uses_sep": ([vp], st),
            "hines_sep_schedule": ([ctypes.c_int32, i32p, i32p, ctypes.c_int32], ctypes.c_int32),
            "hines_sep_multi_layout": ([i64, i32p, i32p, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int32),
            "hines_split_schedule": ([ctypes.c_int32, i32p, i32p, ctypes.c_void_p, ctypes.c_int32],
                                     ctypes.c_int32),
            "hines_plan_destroy": ([vp], st),
            "hines_plan_elems": ([vp], i64),
            "hines_plan_unknowns": ([vp], i64),
            "hines_pack": ([vp, st, vp, vp, vp], st),
            "hines_unpack": ([vp, st, vp, vp, vp], st),
            "hines_work_bytes": ([vp, st], ctypes.c_size_t),
            "hines_solve_batch": ([vp, st, vp, vp, vp, vp, vp, vp, vp], st),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
        return L


def version() -> int:
    return int(load_library().bps_version())


def bps_version() -> int:
    return version()


def bps_init():
    """Prepare the current device (kernel attributes; optional, see bps.h)."""
    _check("bps_init", load_library().bps_init())


def bps_status_str(status: int) -> str:
    return (load_library().bps_status_str(int(status)) or b"").decode()


def bps_last_error() -> str:
    """Message of the last failed call on this thread ('' if none)."""
    return (load_library().bps_last_error() or b"").decode()


def _check(fn: str, status: int):
    if status != 0:
        L = load_library()
        raise BpsError(fn, status, (L.bps_last_error() or b"").decode() or
                       L.bps_status_str(status).decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float64:
        return BPS_F64
    if t.dtype == torch.float32:
        return BPS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected (libbps runs on the GPU only)")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _desc(dtype: int, flags: int, n: int, batch: int, ld: int) -> PentaDesc:
    return PentaDesc(int(dtype), int(flags), int(n), int(batch), int(ld))


def _geom(x, batch):
    if x.dim() != 2:
        raise ValueError("interleaved tensor of shape (n, ld) expected")
    n, ld = x.shape
    return int(n), int(batch if batch is not None else ld), int(ld)


# ---------------------------------------------------------------------------
# Pentadiagonal
# ---------------------------------------------------------------------------

def bps_penta_factor_bytes(n: int, batch: int, ld: int, dtype: int = BPS_F64, flags: int = 0) -> int:
    return int(load_library().bps_penta_factor_bytes(ctypes.byref(_desc(dtype, flags, n, batch, ld))))


def bps_penta_work_bytes(n: int, batch: int, ld: int, dtype: int = BPS_F64,
                         cyclic: bool = False) -> int:
    return int(load_library().bps_penta_work_bytes(
        ctypes.byref(_desc(dtype, BPS_CYCLIC if cyclic else 0, n, batch, ld))))


def _flags(cyclic, shared):
    return (BPS_CYCLIC if cyclic else 0) | (BPS_SHARED_COEF if shared else 0)


def penta_factor_batch(a, b, c, d, e, factors, info=None, *, n=None, batch=None, ld=None,
                       cyclic=False, stream=None):
    """Factor a batch (per-system (n, ld) diagonals, or shared 1-D diagonals).

    For shared diagonals give n/batch/ld of the systems to be solved later
    (only n matters for the factors).  factors: uint8/float device tensor of
    at least bps_penta_factor_bytes bytes.  info: int32 device tensor or None.
    """
    shared = a.dim() == 1
    if shared:
        n = int(a.shape[0]) if n is None else int(n)
        batch = 1 if batch is None else int(batch)
        ld = batch if ld is None else int(ld)
    else:
        n, batch, ld = _geom(a, batch)
    dsc = _desc(_dtype_code(a), _flags(cyclic, shared), n, batch, ld)
    need = load_library().bps_penta_factor_bytes(ctypes.byref(dsc))
    if factors.numel() * factors.element_size() < need:
        raise ValueError(f"factors buffer too small ({need} bytes needed)")
    _check("penta_factor_batch", load_library().penta_factor_batch(
        ctypes.byref(dsc), _ptr(a), _ptr(b), _ptr(c), _ptr(d), _ptr(e), _ptr(factors),
        _ptr(info), _stream(stream)))
    return factors


def penta_solve_batch(factors, x, *, batch=None, shared=False, stream=None):
    """x (n, ld): right-hand sides in, solutions out (non-periodic)."""
    n, batch, ld = _geom(x, batch)
    dsc = _desc(_dtype_code(x), _flags(False, shared), n, batch, ld)
    _check("penta_solve_batch", load_library().penta_solve_batch(
        ctypes.byref(dsc), _ptr(factors), _ptr(x), _stream(stream)))
    return x


def penta_cyclic_solve_batch(factors, x, *, batch=None, shared=False, stream=None):
    """x (n, ld): right-hand sides in, solutions out (periodic)."""
    n, batch, ld = _geom(x, batch)
    dsc = _desc(_dtype_code(x), _flags(True, shared), n, batch, ld)
    _check("penta_cyclic_solve_batch", load_library().penta_cyclic_solve_batch(
        ctypes.byref(dsc), _ptr(factors), _ptr(x), _stream(stream)))
    return x


def penta_factor_solve_batch(a, b, c, d, e, x, work, info=None, *, batch=None, cyclic=False,
                             stream=None):
    """Fused factor + solve, per-system diagonals (n, ld); cyclic: periodic."""
    n, batch, ld = _geom(x, batch)
    dsc = _desc(_dtype_code(x), BPS_CYCLIC if cyclic else 0, n, batch, ld)
    need = load_library().bps_penta_work_bytes(ctypes.byref(dsc))
    if work.numel() * work.element_size() < need:
        raise ValueError(f"work buffer too small ({need} bytes needed)")
    _check("penta_factor_solve_batch", load_library().penta_factor_solve_batch(
        ctypes.byref(dsc), _ptr(a), _ptr(b), _ptr(c), _ptr(d), _ptr(e), _ptr(x), _ptr(work),
        _ptr(info), _stream(stream)))
    return x


# ---------------------------------------------------------------------------
# Hyperdiffusion
# ---------------------------------------------------------------------------

def hyperdiffusion_work_bytes(n: int, batch: int, dtype: int = BPS_F64) -> int:
    return int(load_library().hyperdiffusion_work_bytes(int(dtype), int(n), int(batch)))


def hyperdiffusion_step(C, dt: float, dx: float, nsteps: int, work, diagonals=None, *,
                        batch=None, stream=None):
    """Advance C (n, ld) by nsteps implicit periodic hyperdiffusion steps."""
    n, batch, ld = _geom(C, batch)
    dt_code = _dtype_code(C)
    need = load_library().hyperdiffusion_work_bytes(dt_code, n, batch)
    if work.numel() * work.element_size() < need:
        raise ValueError(f"work buffer too small ({need} bytes needed)")
    _check("hyperdiffusion_step", load_library().hyperdiffusion_step(
        dt_code, n, batch, ld, float(dt), float(dx), _ptr(diagonals), _ptr(C), int(nsteps),
        _ptr(work), _stream(stream)))
    return C


def hyperdiffusion_factor(n: int, dt: float, dx: float, work, diagonals=None, *,
                          dtype: int = BPS_F64, stream=None):
    """Factor the periodic operator (I + sigma D4, or the given diagonals)
    once into work; hyperdiffusion_solve then reuses it."""
    need = load_library().hyperdiffusion_work_bytes(int(dtype), int(n), 1)
    if work.numel() * work.element_size() < need:
        raise ValueError(f"work buffer too small ({need} bytes needed)")
    _check("hyperdiffusion_factor", load_library().hyperdiffusion_factor(
        int(dtype), int(n), float(dt), float(dx), _ptr(diagonals), _ptr(work), _stream(stream)))
    return work


def hyperdiffusion_solve(C, dt: float, dx: float, nsteps: int, work, diagonals=None, *,
                         batch=None, stream=None):
    """Advance C (n, ld) by nsteps steps with the factors of
    hyperdiffusion_factor (same dt, dx, diagonals and dtype)."""
    n, batch, ld = _geom(C, batch)
    dt_code = _dtype_code(C)
    need = load_library().hyperdiffusion_work_bytes(dt_code, n, 1)
    if work.numel() * work.element_size() < need:
        raise ValueError(f"work buffer too small ({need} bytes needed)")
    _check("hyperdiffusion_solve", load_library().hyperdiffusion_solve(
        dt_code, n, batch, ld, float(dt), float(dx), _ptr(diagonals), _ptr(C), int(nsteps),
        _ptr(work), _stream(stream)))
    return C


BPS_NOALLOC_SCRATCH_BYTES = 2 * 1024 * 1024


def hyperdiffusion_step_noalloc(C, dt: float, dx: float, nsteps: int, diagonals=None, *,
                                batch=None, stream=None):
    """hyperdiffusion_step with the library's per-GPU scratch array as work
    memory: allocates nothing (see bps.h for the size limit and the sharing
    of the array between calls on one GPU)."""
    n, batch, ld = _geom(C, batch)
    _check("hyperdiffusion_step_noalloc", load_library().hyperdiffusion_step_noalloc(
        _dtype_code(C), n, batch, ld, float(dt), float(dx), _ptr(diagonals), _ptr(C),
        int(nsteps), _stream(stream)))
    return C


def hyperdiffusion_theta_work_bytes(n: int, batch: int, dtype: int = BPS_F64) -> int:
    return int(load_library().hyperdiffusion_theta_work_bytes(int(dtype), int(n), int(batch)))


def hyperdiffusion_theta_step(C, dt: float, dx: float, theta: float, nsteps: int, work, *,
                              batch=None, stream=None):
    """Advance C (n, ld) by nsteps theta-scheme periodic hyperdiffusion steps."""
    n, batch, ld = _geom(C, batch)
    dt_code = _dtype_code(C)
    need = load_library().hyperdiffusion_theta_work_bytes(dt_code, n, batch)
    if work.numel() * work.element_size() < need:
        raise ValueError(f"work buffer too small ({need} bytes needed)")
    _check("hyperdiffusion_theta_step", load_library().hyperdiffusion_theta_step(
        dt_code, n, batch, ld, float(dt), float(dx), float(theta), _ptr(C), int(nsteps),
        _ptr(work), _stream(stream)))
    return C


def cahn_hilliard_work_bytes(n: int, batch: int, dtype: int = BPS_F64) -> int:
    return int(load_library().cahn_hilliard_work_bytes(int(dtype), int(n), int(batch)))


def cahn_hilliard_step(C, dt: float, dx: float, gamma: float, mobility: float, theta: float,
                       nsteps: int, work, *, batch=None, stream=None):
    """Advance C (n, ld) by nsteps semi-implicit periodic Cahn-Hilliard steps."""
    n, batch, ld = _geom(C, batch)
    dt_code = _dtype_code(C)
    need = load_library().cahn_hilliard_work_bytes(dt_code, n, batch)
    if work.numel() * work.element_size() < need:
        raise ValueError(f"work buffer too small ({need} bytes needed)")
    _check("cahn_hilliard_step", load_library().cahn_hilliard_step(
        dt_code, n, batch, ld, float(dt), float(dx), float(gamma), float(mobility), float(theta),
        _ptr(C), int(nsteps), _ptr(work), _stream(stream)))
    return C


# ---------------------------------------------------------------------------
# Tridiagonal
# ---------------------------------------------------------------------------

def tri_work_bytes(n: int, ld: int, dtype: int = BPS_F64) -> int:
    return int(load_library().tri_work_bytes(int(dtype), int(n), int(ld)))


def tri_solve_batch(a, b, c, y, work, info=None, *, batch=None, stream=None):
    """Solve the tridiagonal systems (a, b, c) u = y in place of y; all
    arrays interleaved (n, ld) on the device, a[0] and c[n-1] ignored."""
    n, batch, ld = _geom(y, batch)
    code = _dtype_code(y)
    for name, v in (("a", a), ("b", b), ("c", c)):
        if tuple(v.shape) != tuple(y.shape) or v.dtype != y.dtype or v.stride() != y.stride():
            raise ValueError(f"{name} must have the shape, dtype and layout of y")
    need = load_library().tri_work_bytes(code, n, ld)
    if work.numel() * work.element_size() < need:
        raise ValueError(f"work buffer too small ({need} bytes needed)")
    _check("tri_solve_batch", load_library().tri_solve_batch(
        code, n, batch, ld, _ptr(a), _ptr(b), _ptr(c), _ptr(y), _ptr(work), _ptr(info),
        _stream(stream)))
    return y


# ---------------------------------------------------------------------------
# Hines
# ---------------------------------------------------------------------------

class HinesPlan:
    """Owns a bps_hines_plan (destroyed on close() / garbage collection)."""

    def __init__(self, handle, batch, mono):
        self._h = handle
        self.batch = int(batch)
        self.mono = bool(mono)

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan already destroyed")
        return self._h

    @property
    def elems(self) -> int:
        return int(load_library().hines_plan_elems(self.handle))

    @property
    def unknowns(self) -> int:
        return int(load_library().hines_plan_unknowns(self.handle))

    @property
    def uses_levels(self) -> bool:
        return bool(load_library().hines_plan_uses_levels(self.handle))

    @property
    def split(self) -> int:
        """Number of trees solved on two lanes."""
        return int(load_library().hines_plan_split(self.handle))

    @property
    def uses_sep(self) -> bool:
        """True when the plan solves with BPS_HINES_SEP (separator schedules)."""
        return bool(load_library().hines_plan_uses_sep(self.handle))

    def close(self):
        if self._h is not None:
            _check("hines_plan_destroy", load_library().hines_plan_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def hines_plan_create(batch: int, sizes, parent, mono: bool, ld: int = 0,
                      schedule: int = BPS_HINES_AUTO) -> HinesPlan:
    """sizes / parent: host int32 arrays (numpy or sequences), see bps.h."""
    import numpy as np
    sz = np.ascontiguousarray(np.asarray(sizes, dtype=np.int32).reshape(-1))
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32).reshape(-1))
    h = ctypes.c_void_p()
    i32p = ctypes.POINTER(ctypes.c_int32)
    _check("hines_plan_create_sched", load_library().hines_plan_create_sched(
        ctypes.byref(h), int(batch), sz.ctypes.data_as(i32p), par.ctypes.data_as(i32p),
        1 if mono else 0, int(ld), int(schedule)))
    return HinesPlan(h, batch, mono)


def hines_plan_create_sched(batch: int, sizes, parent, mono: bool, ld: int = 0,
                            schedule: int = BPS_HINES_AUTO) -> HinesPlan:
    """hines_plan_create with an explicit schedule (BPS_HINES_*)."""
    return hines_plan_create(batch, sizes, parent, mono, ld, schedule)


def hines_plan_elems(plan: HinesPlan) -> int:
    return plan.elems


def hines_plan_unknowns(plan: HinesPlan) -> int:
    return plan.unknowns


def hines_plan_split(plan: HinesPlan) -> int:
    return plan.split


def hines_split_schedule(parent):
    """Host-only two-lane schedule of one tree (see bps.h): (node, code), each
    of shape (2, rows), or None when the tree stays on one lane."""
    import numpy as np
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32).reshape(-1))
    n = len(par)
    cap = 2 * n + 80
    node = np.empty(2 * cap, dtype=np.int32)
    code = np.empty(2 * cap, dtype=np.uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    L = load_library()
    m = L.hines_split_schedule(n, par.ctypes.data_as(i32p), node.ctypes.data_as(i32p),
                               code.ctypes.data_as(ctypes.c_void_p), cap)
    if m < 0:
        raise BpsError("hines_split_schedule", 1, (L.bps_last_error() or b"").decode())
    if m == 0:
        return None
    return node.reshape(2, cap)[:, :m].copy(), code.reshape(2, cap)[:, :m].copy()


def hines_plan_uses_levels(plan: HinesPlan) -> bool:
    return plan.uses_levels


def hines_plan_uses_sep(plan: HinesPlan) -> bool:
    return plan.uses_sep


def hines_sep_multi_layout(sizes, parent):
    """Host-only BPS_HINES_SEP layout of a multi-morphology batch (see bps.h):
    a dict with nwg, elems, R, lds, K (lanes per workgroup), code, comp, pos,
    lanetab (nwg*K, 5), wgoff, tabs; None when the batch does not qualify."""
    import numpy as np
    sz = np.ascontiguousarray(np.asarray(sizes, dtype=np.int32).reshape(-1))
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32).reshape(-1))
    i32p = ctypes.POINTER(ctypes.c_int32)
    L = load_library()
    dims = np.zeros(6, dtype=np.int64)
    st = L.hines_sep_multi_layout(len(sz), sz.ctypes.data_as(i32p), par.ctypes.data_as(i32p),
                                  dims.ctypes.data, None, None, None, None, None, None)
    if st < 0:
        raise BpsError("hines_sep_multi_layout", 1, (L.bps_last_error() or b"").decode())
    if st == 0:
        return None
    nwg, elems, R, lds, ntab, K = (int(v) for v in dims)
    code = np.zeros(elems, dtype=np.uint16)
    comp = np.zeros(elems, dtype=np.int32)
    pos = np.zeros(int(sz.sum()), dtype=np.int32)
    lanetab = np.zeros(nwg * K * 5, dtype=np.int32)
    wgoff = np.zeros(nwg + 1, dtype=np.int64)
    tabs = np.zeros(max(ntab, 1), dtype=np.int32)
    st = L.hines_sep_multi_layout(len(sz), sz.ctypes.data_as(i32p), par.ctypes.data_as(i32p),
                                  dims.ctypes.data, code.ctypes.data, comp.ctypes.data, pos.ctypes.data,
                                  lanetab.ctypes.data, wgoff.ctypes.data, tabs.ctypes.data)
    if st != 1:
        raise BpsError("hines_sep_multi_layout", 1, (L.bps_last_error() or b"").decode())
    return {"nwg": nwg, "elems": elems, "R": R, "lds": lds, "K": K, "code": code, "comp": comp,
            "pos": pos, "lanetab": lanetab.reshape(nwg * K, 5), "wgoff": wgoff, "tabs": tabs}


def hines_sep_schedule(parent):
    """Host-only BPS_HINES_SEP schedule of one tree (see bps.h), decoded:
    a dict with R, lanes (16, 32 or 64), neurons (per workgroup), ns, nc,
    npc, nh, codes (lanes, R)
    uint32, bases (lanes, 3), septab (ns, 5), comptab (nc, 3), clist (nc,);
    None when the tree does not qualify."""
    import numpy as np
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32).reshape(-1))
    n = len(par)
    cap = 8 + 64 * 32 + 64 * 3 + 5 * n + 4 * n + 64
    out = np.zeros(cap, dtype=np.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    L = load_library()
    m = L.hines_sep_schedule(n, par.ctypes.data_as(i32p), out.ctypes.data_as(i32p), cap)
    if m < 0:
        raise BpsError("hines_sep_schedule", 1, (L.bps_last_error() or b"").decode())
    if m == 0:
        return None
    R, ns, nc, npc, nh = (int(v) for v in out[:5])
    K = int(out[6])
    o = 8
    codes = out[o:o + K * R].view(np.uint32).reshape(K, R).copy()
    o += K * R
    bases = out[o:o + 3 * K].reshape(K, 3).copy()
    o += 3 * K
    septab = out[o:o + ns * 5].reshape(ns, 5).copy()
    o += ns * 5
    comptab = out[o:o + nc * 3].reshape(nc, 3).copy()
    o += nc * 3
    clist = out[o:o + nc].copy()
    return {"R": R, "lanes": K, "neurons": int(out[7]), "ns": ns, "nc": nc, "npc": npc, "nh": nh,
            "codes": codes, "bases": bases,
            "septab": septab, "comptab": comptab, "clist": clist}


def hines_plan_destroy(plan: HinesPlan):
    plan.close()


def _hines_sizes(plan, flat, packed):
    if flat.numel() < plan.unknowns:
        raise ValueError(f"flat array too small ({plan.unknowns} values needed)")
    if packed.numel() < plan.elems:
        raise ValueError(f"packed array too small ({plan.elems} values needed)")
    if flat.dtype != packed.dtype:
        raise ValueError("flat and packed arrays must have the same dtype")


def hines_pack(plan: HinesPlan, flat, packed, stream=None):
    _hines_sizes(plan, flat, packed)
    _check("hines_pack", load_library().hines_pack(plan.handle, _dtype_code(flat), _ptr(flat),
                                                   _ptr(packed), _stream(stream)))
    return packed


def hines_unpack(plan: HinesPlan, packed, flat, stream=None):
    _hines_sizes(plan, flat, packed)
    _check("hines_unpack", load_library().hines_unpack(plan.handle, _dtype_code(packed),
                                                       _ptr(packed), _ptr(flat), _stream(stream)))
    return flat


def hines_work_bytes(plan: HinesPlan, dtype: int = BPS_F64) -> int:
    return int(load_library().hines_work_bytes(plan.handle, int(dtype)))


def hines_solve_batch(plan: HinesPlan, u, l, d, rhs, work, info=None, stream=None):
    """rhs: right-hand sides in, voltages out (solver layout of the plan)."""
    _check("hines_solve_batch", load_library().hines_solve_batch(
        plan.handle, _dtype_code(rhs), _ptr(u), _ptr(l), _ptr(d), _ptr(rhs), _ptr(work),
        _ptr(info), _stream(stream)))
    return rhs
