"""Helpers for the GPU tests: device transfers and the parity metric."""
import numpy as np
import torch

import banded_pde_solvers_amd as bps

DEV = "cuda:0"
TOL = {torch.float64: 1e-10, torch.float32: 1e-4}


def dev(x, dtype=torch.float64):
    return torch.as_tensor(np.ascontiguousarray(x)).to(device=DEV, dtype=dtype)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().to(torch.float64).numpy()


def relerr_cols(x, y):
    """Per-system (column) normwise relative error of interleaved (n, batch)."""
    num = np.linalg.norm(x - y, axis=0)
    den = np.linalg.norm(y, axis=0)
    return float(np.max(num / den))


def buf(nbytes):
    return torch.empty(max(int(nbytes), 8), dtype=torch.uint8, device=DEV)


def info_buf(k):
    return torch.full((k,), -7, dtype=torch.int32, device=DEV)


def rounded(x, dtype):
    """Values as the GPU sees them in `dtype`, promoted back to float64."""
    return np.asarray(x).astype(np.float32).astype(np.float64) if dtype == torch.float32 else x
