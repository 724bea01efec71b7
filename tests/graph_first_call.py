"""Child process of test_gpu_graphs.test_first_call_inside_capture.

In a fresh process, the first call of the library on the device -- a chunked
fp64 pentadiagonal factor+solve whose kernel needs 80 KiB of dynamic LDS, so
that call also sets the kernel attributes of the device -- is made inside a
HIP graph capture (torch's global capture mode, which rejects unsafe calls).
The graph is replayed three times, each result compared bit for bit with an
eager call made afterwards, and that result with the oracle."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import banded_pde_solvers_amd as bps  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402


def main():
    n, batch = 512, 100
    print(f"first captured call: penta_factor_solve_batch n={n} batch={batch} fp64", flush=True)
    pb = W.penta_dominant(n, batch, rng=np.random.default_rng(5))
    dg = [torch.as_tensor(v, device="cuda:0") for v in pb.diagonals]
    x0 = torch.as_tensor(pb.f, device="cuda:0")
    x = x0.clone()
    work = torch.empty(bps.bps_penta_work_bytes(n, batch, batch), dtype=torch.uint8,
                       device="cuda:0")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bps.penta_factor_solve_batch(*dg, x, work)
    outs = []
    for _ in range(3):
        x.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        outs.append(x.cpu().numpy())
    x.copy_(x0)
    bps.penta_factor_solve_batch(*dg, x, work)
    torch.cuda.synchronize()
    eager = x.cpu().numpy()
    for o in outs:
        np.testing.assert_array_equal(o, eager)
    xr, _ = oracle.penta_solve(*(W.to_flat(v) for v in (*pb.diagonals, pb.f)))
    xr = W.to_interleaved(xr)
    err = float(np.max(np.linalg.norm(eager - xr, axis=0) / np.linalg.norm(xr, axis=0)))
    assert err <= 1e-10, err
    print(f"FIRST_CALL_CAPTURE_OK rel err {err:.2e}", flush=True)


if __name__ == "__main__":
    main()
