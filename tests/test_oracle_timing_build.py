"""The CPU-baseline timing build of the oracle (gcc -O3 -march=native, no
contraction, no fast-math) computes what the checker build computes: bit
for bit on each method, so the baseline times the oracle as it stands."""
import subprocess
import sys

import numpy as np

import workloads as W

SCRIPT = r"""
import sys, numpy as np
sys.path.insert(0, {root!r})
import oracle, workloads as W
if {timing}:
    oracle.use_library(oracle.build_timing({tmp!r}))
rng = np.random.default_rng(5)
out = []
pb = W.penta_dominant(64, 9, rng=rng)
out.append(oracle.penta_solve(*(W.to_flat(v) for v in (*pb.diagonals, pb.f)))[0])
pc = W.penta_dominant(48, 7, cyclic=True, rng=rng)
out.append(oracle.penta_solve(*(W.to_flat(v) for v in (*pc.diagonals, pc.f)), cyclic=True)[0])
out.append(oracle.hyperdiffusion(rng.uniform(-1, 1, (5, 128)), 1e-6, 1 / 128, 4))
out.append(oracle.hyperdiffusion_theta(rng.uniform(-1, 1, (5, 96)), 1e-6, 1 / 96, 0.5, 3))
hm = W.hines_mono(77, 6, rng=rng)
out.append(oracle.hines_solve(hm.parent, *(W.to_flat(v) for v in (hm.u, hm.l, hm.d, hm.rhs)))[0])
tb = W.tri_dominant(40, 6, rng=rng)
out.append(oracle.thomas_solve(*(W.to_flat(v) for v in (tb.a, tb.b, tb.c, tb.y)))[0])
np.savez({npz!r}, *out)
"""


def _run(tmp_path, timing):
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    npz = str(tmp_path / ("timing.npz" if timing else "checker.npz"))
    code = SCRIPT.format(root=root, timing=timing, tmp=str(tmp_path), npz=npz)
    subprocess.check_call([sys.executable, "-c", code])
    with np.load(npz) as z:
        return [z[k] for k in sorted(z.files, key=lambda s: int(s.split("_")[1]))]


def test_timing_build_equals_checker_build(tmp_path):
    a = _run(tmp_path, False)
    b = _run(tmp_path, True)
    assert len(a) == len(b) == 6
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
