#!/usr/bin/env python3
"""Benchmark of the batched banded-solver hot path on one MI355X.

Default workload (the headline): periodic hyperdiffusion with constant
coefficients, N = 1024 unknowns per system, 16384 systems, fp64,
sigma = dt/dx^4 with dt = 1e-6, dx = 1/1024, 100 implicit time steps per
benchmark step.  One benchmark step is one hyperdiffusion_step call: build
the operator, factor it once (with the periodic-reduction quantities), and
run all 100 solves (forward sweep, corner solve, backward sweep) on every
system -- the whole path on one batch of synthetic input already resident in
device memory.

Output: ONE JSON line (metric, value = unknowns solved per second, ...),
with a "roofline" object for the dominant kernel (the multi-step periodic
solve; algorithmic bytes = 16 per unknown per time step: read C^k, write
C^{k+1}) and a "cpu_baseline" object (the CPU oracle, OpenMP over systems,
timed on a bounded sample of the same workload on this host's cores).

    python bench.py [--steps K] [--warmup W] [--workload {1,2,3,4}]

--workload selects another workload for manual measurements
(2: general pentadiagonal 512 x 65536 fused factor+solve; 3: Hines mono
512 x 100000; 4: Hines multi, 32768 neurons of 256..2048 compartments,
20 solves per step).  Only one GPU is used; --gpus above 1 exits.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E peak, GB/s
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _time_loop(fn, steps, warmup):
    """Warm up, then time exactly `steps` calls bracketed by synchronisation;
    also record each call with HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [_events() for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in evs]
    return wall, per


def _traffic(kernel):
    try:
        with open(PROFILE_TRAFFIC) as fh:
            return json.load(fh).get(kernel)
    except (OSError, ValueError):
        return None


def _cpu_baseline(run_sample, unknowns_per_system, label, seconds):
    """Time the oracle on a growing sample until it takes ~`seconds`."""
    import oracle
    cores = oracle.set_threads(0)
    k = 8
    t = 0.0
    while True:
        t0 = time.perf_counter()
        run_sample(k)
        t = time.perf_counter() - t0
        if t >= seconds / 4 or k >= 1 << 20:
            break
        k = int(k * min(16.0, max(2.0, seconds / 4 / max(t, 1e-4))))
    # final timed sample sized to ~seconds
    k = max(1, int(k * seconds / max(t, 1e-6) / 2))
    t0 = time.perf_counter()
    run_sample(k)
    t = time.perf_counter() - t0
    return {"value": k * unknowns_per_system / t, "unit": "unknowns/s", "cores": cores,
            "kind": "oracle", "sample": f"{k} {label} in {t:.2f} s"}


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def bench_hyperdiffusion(args):
    import numpy as np
    import torch
    import banded_pde_solvers_amd as bps
    import workloads as W

    cfg = W.WORKLOADS[1]
    n, batch, nsteps, dt, dx = cfg["n"], cfg["batch"], cfg["nsteps"], cfg["dt"], cfg["dx"]
    C = torch.as_tensor(W.hyperdiffusion_random(n, batch), device="cuda:0")
    work = torch.empty(bps.hyperdiffusion_work_bytes(n, batch), dtype=torch.uint8, device="cuda:0")
    step = lambda: bps.hyperdiffusion_step(C, dt, dx, nsteps, work)
    wall, per = _time_loop(step, args.steps, args.warmup)
    # the operator set-up alone (diagonals + shared factorisation), same stream
    _, setup = _time_loop(lambda: bps.hyperdiffusion_step(C, dt, dx, 0, work), 10, 2)
    ms_step = wall * 1e3 / args.steps
    kern_ms = max(statistics.mean(per) - statistics.median(setup), 1e-6)
    unknowns = n * batch * nsteps
    alg_bytes = 16.0 * unknowns                      # read C^k + write C^{k+1}, fp64
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    line = {
        "metric": "unknowns solved/s (fp64), periodic hyperdiffusion implicit steps",
        "value": unknowns / (ms_step * 1e-3),
        "unit": "unknowns/s",
        "ms_per_step": ms_step,
        "dtype": "f64",
        "config": {"workload": cfg["name"], "n": n, "batch": batch, "time_steps_per_step": nsteps,
                   "dt": dt, "dx": dx, "sigma": dt / dx ** 4, "coefficients": "constant (factor once)"},
        "roofline": {"bound": "hbm", "kernel": "k_penta_cyclic_solve<double,shared>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": _traffic("hyperdiffusion"),
                     "kernel_ms": kern_ms, "setup_ms": statistics.median(setup),
                     "bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        C0 = W.hyperdiffusion_random(n, 2048, rng=np.random.default_rng(77))

        def sample(k):
            reps = (k + 2047) // 2048
            for r in range(reps):
                kk = min(2048, k - r * 2048)
                oracle.hyperdiffusion(W.to_flat(C0[:, :kk]), dt, dx, nsteps)
        line["cpu_baseline"] = _cpu_baseline(sample, n * nsteps, f"systems x {nsteps} steps",
                                             args.cpu_seconds)
    return line


def bench_penta(args):
    import numpy as np
    import torch
    import banded_pde_solvers_amd as bps
    import workloads as W

    cfg = W.WORKLOADS[2]
    n, batch = cfg["n"], cfg["batch"]
    dt = torch.float32 if args.dtype == "f32" else torch.float64
    pb = W.penta_dominant(n, batch)
    dg = [torch.as_tensor(v, device="cuda:0").to(dt) for v in pb.diagonals]
    f0 = torch.as_tensor(pb.f, device="cuda:0").to(dt)
    x = f0.clone()
    code = bps.BPS_F32 if dt == torch.float32 else bps.BPS_F64
    work = torch.empty(bps.bps_penta_work_bytes(n, batch, batch, code), dtype=torch.uint8,
                       device="cuda:0")
    del pb

    def step():
        bps.penta_factor_solve_batch(*dg, x, work)
    wall, per = _time_loop(step, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    es = 4 if dt == torch.float32 else 8
    unknowns = n * batch
    alg_bytes = 7.0 * es * unknowns                  # 5 diagonals + f in, x out
    kern_ms = statistics.mean(per)
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    line = {
        "metric": f"unknowns solved/s ({args.dtype}), general pentadiagonal factor+solve",
        "value": unknowns / (ms_step * 1e-3), "unit": "unknowns/s", "ms_per_step": ms_step,
        "dtype": args.dtype,
        "config": {"workload": cfg["name"], "n": n, "batch": batch, "coefficients": "per system"},
        "roofline": {"bound": "hbm", "kernel": "k_penta_fused", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": _traffic("penta_fused_" + args.dtype), "kernel_ms": kern_ms,
                     "bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        small = W.penta_dominant(n, 4096, rng=np.random.default_rng(5))
        fl = [W.to_flat(v) for v in (*small.diagonals, small.f)]

        def sample(k):
            for r in range((k + 4095) // 4096):
                kk = min(4096, k - r * 4096)
                oracle.penta_solve(*(v[:kk] for v in fl))
        line["cpu_baseline"] = _cpu_baseline(sample, n, "systems", args.cpu_seconds)
    return line


def _hines_common(args, multi):
    import numpy as np
    import torch
    import banded_pde_solvers_amd as bps
    import workloads as W

    cfg = W.WORKLOADS[4 if multi else 3]
    if multi:
        mm = W.hines_multi(cfg["batch"], cfg["nmin"], cfg["nmax"])
        plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False)
        arrs = []
        for v in (mm.u, mm.l, mm.d, mm.rhs):
            t = torch.empty(plan.elems, dtype=torch.float64, device="cuda:0")
            bps.hines_pack(plan, torch.as_tensor(v, device="cuda:0"), t)
            arrs.append(t)
        nsolve = cfg["nsteps"]
        stats = {"mean_n": float(mm.sizes.mean()), "padded_elems": plan.elems}
    else:
        hm = W.hines_mono(cfg["n"], cfg["batch"])
        plan = bps.hines_plan_create(cfg["batch"], [cfg["n"]], hm.parent, mono=True)
        arrs = [torch.as_tensor(v, device="cuda:0") for v in (hm.u, hm.l, hm.d, hm.rhs)]
        nsolve = 1
        stats = W.tree_stats(hm.parent)
    u, l, d, rhs = arrs
    work = torch.empty(bps.hines_work_bytes(plan), dtype=torch.uint8, device="cuda:0")

    def step():
        for _ in range(nsolve):          # rhs_{k+1} = V_k, d restored (kept constant)
            bps.hines_solve_batch(plan, u, l, d, rhs, work)
    wall, per = _time_loop(step, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    unknowns = plan.unknowns * nsolve
    per_unknown = 44.0 if multi else 40.0            # u, l, d, rhs in, V out (+ parent)
    alg_bytes = per_unknown * unknowns
    kern_ms = statistics.mean(per) / nsolve
    achieved = per_unknown * plan.unknowns / (kern_ms * 1e-3) / 1e9
    line = {
        "metric": "unknowns solved/s (fp64), Hines " + ("multi" if multi else "mono"),
        "value": unknowns / (ms_step * 1e-3), "unit": "unknowns/s", "ms_per_step": ms_step,
        "dtype": "f64",
        "config": {"workload": cfg["name"], "solves_per_step": nsolve, **stats},
        "roofline": {"bound": "hbm", "kernel": "k_hines", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": _traffic("hines_multi" if multi else "hines_mono"),
                     "kernel_ms": kern_ms, "bytes_per_launch": alg_bytes / nsolve},
    }
    if not args.no_cpu_baseline:
        import oracle
        if multi:
            small = W.hines_multi(2048, cfg["nmin"], cfg["nmax"], rng=np.random.default_rng(9))

            def sample(k):
                for r in range((k + 2047) // 2048):
                    kk = min(2048, k - r * 2048)
                    o = small.offsets[:kk + 1]
                    e = o[-1]
                    oracle.hines_multi_solve(o, small.parent[:e], small.u[:e], small.l[:e],
                                             small.d[:e], small.rhs[:e])
            line["cpu_baseline"] = _cpu_baseline(sample, float(small.sizes.mean()), "neurons",
                                                 args.cpu_seconds)
        else:
            small = W.hines_mono(cfg["n"], 4096, rng=np.random.default_rng(9))
            fl = [W.to_flat(v) for v in (small.u, small.l, small.d, small.rhs)]

            def sample(k):
                for r in range((k + 4095) // 4096):
                    kk = min(4096, k - r * 4096)
                    oracle.hines_solve(small.parent, *(v[:kk] for v in fl))
            line["cpu_baseline"] = _cpu_baseline(sample, cfg["n"], "neurons", args.cpu_seconds)
    plan.close()
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1, choices=[1, 2, 3, 4])
    ap.add_argument("--dtype", default="f64", choices=["f64", "f32"], help="workload 2 only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: the solver batches are independent and "
                  "this build runs on a single MI355X (see DESIGN.md for how the batch would "
                  "shard); rerun with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import banded_pde_solvers_amd as bps
    bps.load_library()
    fn = {1: bench_hyperdiffusion, 2: bench_penta, 3: lambda a: _hines_common(a, False),
          4: lambda a: _hines_common(a, True)}[args.workload]
    line = fn(args)
    out = {"metric": line.pop("metric"), "value": line.pop("value"), "unit": line.pop("unit"),
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": line.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": line.pop("dtype"), "data": "synthetic (seeded)",
           "config": line.pop("config")}
    out.update(line)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
