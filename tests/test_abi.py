"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, answers size queries, and rejects invalid arguments on the
host (BPS_EINVAL / BPS_ENOTSUP) before anything is enqueued.  No call here
reaches a kernel launch: every case fails validation first."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import banded_pde_solvers_amd as bps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bps.h")

EINVAL, ENOTSUP = 1, 2


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"(?m)^BPS_API\s+[\w\s\*]*?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bps.library_path()):
        pytest.fail("libbps.so is not built (run __graft_entry__.build())")
    return bps.load_library()


def test_header_declares_the_entry_points():
    names = _declared()
    for required in ("penta_factor_batch", "penta_solve_batch", "penta_cyclic_solve_batch",
                     "penta_factor_solve_batch", "hines_solve_batch", "hyperdiffusion_step",
                     "hyperdiffusion_theta_step", "cahn_hilliard_step", "tri_solve_batch",
                     "hines_plan_create", "hines_plan_destroy", "hines_pack", "hines_unpack",
                     "hines_plan_create_sched", "hines_plan_uses_levels"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", bps.library_path()], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        assert getattr(lib, n) is not None


def test_status_strings_and_version(lib):
    assert lib.bps_status_str(0) == b"BPS_OK"
    assert b"invalid" in lib.bps_status_str(EINVAL)
    assert bps.version() >= 100


def test_size_queries(lib):
    F64, F32 = bps.BPS_F64, bps.BPS_F32
    assert bps.bps_penta_factor_bytes(512, 100, 128, F64) == 5 * 512 * 128 * 8
    assert bps.bps_penta_factor_bytes(512, 100, 100, F32, bps.BPS_SHARED_COEF) == 5 * 512 * 4
    assert bps.bps_penta_factor_bytes(10, 3, 3, F64, bps.BPS_CYCLIC) == (9 * 8 + 4) * 3 * 8
    assert bps.bps_penta_factor_bytes(3, 1, 1, F64) == 0          # n < 4
    assert bps.bps_penta_factor_bytes(5, 1, 1, F64, bps.BPS_CYCLIC) == 0   # periodic needs n >= 6
    assert bps.bps_penta_work_bytes(512, 10, 16, F64) == 2 * 512 * 16 * 8
    assert bps.hyperdiffusion_work_bytes(1024, 16384, F64) == (5 * 1024 + 9 * 1022 + 4) * 8
    assert bps.hyperdiffusion_work_bytes(5, 1, F64) == 0


def _desc(dtype=2, flags=0, n=8, batch=4, ld=4):
    return ctypes.byref(bps.PentaDesc(dtype, flags, n, batch, ld))


def _fake(k=0):
    # an aligned non-NULL address; validation rejects these calls before use
    return ctypes.c_void_p(4096 + 64 * k)


@pytest.mark.parametrize("kw,code", [
    (dict(n=3), EINVAL), (dict(batch=0), EINVAL), (dict(ld=3, batch=4), EINVAL),
    (dict(dtype=7), EINVAL), (dict(flags=0x10), EINVAL), (dict(flags=1, n=5), EINVAL),
    (dict(n=1 << 20, ld=1 << 21), EINVAL),          # n * ld above 2^40 elements
    (dict(n=8, ld=1 << 62), EINVAL),                # and no overflow on the way
])
def test_penta_factor_rejects_bad_desc(lib, kw, code):
    st = lib.penta_factor_batch(_desc(**kw), *(_fake(i) for i in range(6)), None, None)
    assert st == code
    assert lib.bps_last_error()


def test_null_and_misaligned_pointers_rejected(lib):
    args = [_fake(i) for i in range(6)]
    args[2] = None
    assert lib.penta_factor_batch(_desc(), *args, None, None) == EINVAL
    assert b"c is NULL" in lib.bps_last_error()
    args[2] = ctypes.c_void_p(4096 + 4)     # not 8-byte aligned for F64
    assert lib.penta_factor_batch(_desc(), *args, None, None) == EINVAL
    assert b"aligned" in lib.bps_last_error()
    assert lib.penta_solve_batch(_desc(), None, _fake(), None) == EINVAL
    assert lib.penta_solve_batch(None, _fake(), _fake(), None) == EINVAL


def test_solve_kind_mismatch_rejected(lib):
    assert lib.penta_solve_batch(_desc(flags=1), _fake(), _fake(1), None) == EINVAL
    assert lib.penta_cyclic_solve_batch(_desc(flags=0), _fake(), _fake(1), None) == EINVAL
    for flags in (2, 3):           # shared coefficients: not a fused use
        assert lib.penta_factor_solve_batch(_desc(flags=flags), *(_fake(i) for i in range(8)),
                                            None, None) == ENOTSUP


def test_hyperdiffusion_rejects_bad_arguments(lib):
    f = lib.hyperdiffusion_step
    assert f(2, 5, 4, 4, 1e-6, 0.1, None, _fake(), 1, _fake(1), None) == EINVAL   # n < 6
    assert f(2, 16, 4, 4, 1e-6, 0.0, None, _fake(), 1, _fake(1), None) == EINVAL  # dx = 0
    assert f(2, 16, 4, 4, float("nan"), 0.1, None, _fake(), 1, _fake(1), None) == EINVAL
    assert f(2, 16, 4, 4, 1e-6, 0.1, None, _fake(), -1, _fake(1), None) == EINVAL
    assert f(2, 16, 4, 3, 1e-6, 0.1, None, _fake(), 1, _fake(1), None) == EINVAL  # ld < batch
    assert f(2, 16, 4, 4, 1e-6, 0.1, None, None, 1, _fake(1), None) == EINVAL


def test_tri_rejects_bad_arguments(lib):
    f = lib.tri_solve_batch
    p = [_fake(i) for i in range(5)]
    assert f(3, 16, 4, 4, *p, None, None) == EINVAL          # dtype
    assert f(2, 0, 4, 4, *p, None, None) == EINVAL           # n < 1
    assert f(2, 16, 0, 4, *p, None, None) == EINVAL          # batch < 1
    assert f(2, 16, 5, 4, *p, None, None) == EINVAL          # ld < batch
    assert f(2, 16, 4, 4, None, *p[1:], None, None) == EINVAL
    assert f(2, 16, 4, 4, *p[:4], None, None, None) == EINVAL   # work
    assert f(2, 16, 4, 4, ctypes.c_void_p(12), *p[1:], None, None) == EINVAL   # misaligned
    assert lib.tri_work_bytes(2, 100, 37) == 100 * 37 * 8
    assert lib.tri_work_bytes(1, 100, 37) == 100 * 37 * 4
    assert lib.tri_work_bytes(2, 0, 37) == 0


def test_cahn_hilliard_rejects_bad_arguments(lib):
    f = lib.cahn_hilliard_step
    ok = (2, 16, 4, 4, 1e-6, 0.1, 1e-4, 1.0, 1.0, _fake(), 1, _fake(1), None)

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[{"n": 1, "dx": 5, "gamma": 6, "mob": 7, "theta": 8, "nsteps": 10}[k]] = v
        return f(*args)
    assert call(gamma=-1e-4) == EINVAL
    assert call(gamma=float("inf")) == EINVAL
    assert call(mob=float("nan")) == EINVAL
    assert call(mob=-1.0) == EINVAL
    assert call(theta=1.01) == EINVAL
    assert call(n=5) == EINVAL
    assert call(dx=0.0) == EINVAL
    assert call(nsteps=-2) == EINVAL
    assert lib.cahn_hilliard_work_bytes(2, 1024, 100) == lib.hyperdiffusion_theta_work_bytes(2, 1024, 100)
    assert lib.cahn_hilliard_work_bytes(1, 4, 3) == 0


def test_theta_step_rejects_bad_arguments(lib):
    f = lib.hyperdiffusion_theta_step
    assert f(2, 16, 4, 4, 1e-6, 0.1, -0.1, _fake(), 1, _fake(1), None) == EINVAL   # theta < 0
    assert f(2, 16, 4, 4, 1e-6, 0.1, 1.5, _fake(), 1, _fake(1), None) == EINVAL    # theta > 1
    assert f(2, 16, 4, 4, 1e-6, 0.1, float("nan"), _fake(), 1, _fake(1), None) == EINVAL
    assert f(2, 5, 4, 4, 1e-6, 0.1, 0.5, _fake(), 1, _fake(1), None) == EINVAL     # n < 6
    assert f(2, 16, 4, 4, 1e-6, 0.0, 0.5, _fake(), 1, _fake(1), None) == EINVAL    # dx = 0
    assert f(2, 16, 4, 4, 1e-6, 0.1, 0.5, _fake(), -1, _fake(1), None) == EINVAL   # nsteps < 0
    assert lib.hyperdiffusion_theta_work_bytes(2, 1024, 100) == (
        lib.hyperdiffusion_work_bytes(2, 1024, 100) + 1024 * 100 * 8)
    assert lib.hyperdiffusion_theta_work_bytes(2, 5, 1) == 0


def test_hines_plan_rejects_bad_parents_before_allocating(lib):
    with pytest.raises(bps.BpsError) as ei:
        bps.hines_plan_create(10, [4], [-1, 0, 2, 1], mono=True)      # parent[2] = 2
    assert ei.value.status == EINVAL
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(2, [3, 2], [-1, 0, 0, -1, 1], mono=False)  # neuron 1: parent[1]=1
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(4, [0], [0], mono=True)                  # n < 1
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(4, [3], [-1, 0, 1], mono=True, ld=2)     # ld < batch


def test_hines_plan_rejects_unknown_schedule(lib):
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(4, [3], [-1, 0, 1], mono=True, schedule=3)
    assert lib.hines_plan_uses_levels(None) == 0


def test_hines_solve_rejects_null_plan_and_dtype(lib):
    assert lib.hines_solve_batch(None, 2, *(_fake(i) for i in range(5)), None, None) == EINVAL
    assert lib.hines_work_bytes(None, 2) == 0


def test_binding_rejects_undersized_work_before_any_call():
    """The Python wrappers compare the work buffer with the library's size
    query and raise before the C call (the C ABI cannot see buffer sizes)."""
    import torch
    small = torch.empty(8, dtype=torch.uint8)
    C = torch.zeros(64, 4, dtype=torch.float64)
    with pytest.raises(ValueError):
        bps.hyperdiffusion_theta_step(C, 1e-6, 1 / 64, 0.5, 1, small)
    with pytest.raises(ValueError):
        bps.cahn_hilliard_step(C, 1e-6, 1 / 64, 1e-4, 1.0, 1.0, 1, small)
    with pytest.raises(ValueError):
        bps.tri_solve_batch(C, C, C, C, small)
    with pytest.raises(ValueError):
        bps.penta_factor_solve_batch(C, C, C, C, C, C, small, cyclic=True)


def test_binding_has_every_declared_entry_point():
    """The Python binding exposes each C entry point of bps.h under its name."""
    names = _declared()
    missing = sorted(n for n in names if not hasattr(bps, n))
    assert not missing, missing
    assert bps.bps_status_str(1).startswith("BPS_EINVAL")
    assert bps.bps_version() == bps.version()


def test_hyperdiffusion_factor_solve_and_noalloc_reject_bad_arguments(lib):
    """The two halves of hyperdiffusion_step and its allocation-free variant
    validate like the step itself; the allocation-free call rejects sizes
    whose work exceeds its scratch array before touching the device."""
    fa, so, na = lib.hyperdiffusion_factor, lib.hyperdiffusion_solve, lib.hyperdiffusion_step_noalloc
    assert fa(2, 5, 1e-6, 0.1, None, _fake(), None) == EINVAL            # n < 6
    assert fa(2, 16, 1e-6, 0.0, None, _fake(), None) == EINVAL           # dx = 0
    assert fa(2, 16, float("inf"), 0.1, None, _fake(), None) == EINVAL
    assert fa(2, 16, 1e-6, 0.1, None, None, None) == EINVAL              # work
    assert fa(3, 16, 1e-6, 0.1, None, _fake(), None) == EINVAL           # dtype
    assert fa(2, 16, 1e-6, 0.1, ctypes.c_void_p(4096 + 4), _fake(), None) == EINVAL
    assert so(2, 16, 4, 3, 1e-6, 0.1, None, _fake(), 1, _fake(1), None) == EINVAL   # ld
    assert so(2, 16, 4, 4, 1e-6, 0.1, None, _fake(), -2, _fake(1), None) == EINVAL  # nsteps
    assert so(2, 16, 4, 4, 1e-6, 0.1, None, _fake(), 1, None, None) == EINVAL       # work
    assert so(2, 16, 4, 4, 1e-6, 0.1, None, None, 1, _fake(1), None) == EINVAL      # C
    assert na(2, 5, 4, 4, 1e-6, 0.1, None, _fake(), 1, None) == EINVAL              # n < 6
    assert na(2, 16, 4, 4, 1e-6, 0.1, None, None, 1, None) == EINVAL                # C
    for dtype, n in ((2, 18726), (1, 37451)):
        assert na(dtype, n, 2, 2, 1e-6, 1.0 / n, None, _fake(), 1, None) == EINVAL
        assert b"scratch" in lib.bps_last_error()
    # the largest sizes fit the array
    assert bps.hyperdiffusion_work_bytes(18725, 1, 2) <= bps.BPS_NOALLOC_SCRATCH_BYTES
    assert bps.hyperdiffusion_work_bytes(37450, 1, 1) <= bps.BPS_NOALLOC_SCRATCH_BYTES
    assert bps.hyperdiffusion_work_bytes(18726, 1, 2) > bps.BPS_NOALLOC_SCRATCH_BYTES


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define BPS_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", text)
    assert m and int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == bps.BPS_NOALLOC_SCRATCH_BYTES
