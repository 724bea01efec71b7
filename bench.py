#!/usr/bin/env python3
"""Benchmark of the batched banded-solver hot path on one MI355X.

Default workload (the headline): periodic hyperdiffusion with constant
coefficients, N = 1024 unknowns per system, 16384 systems, fp64,
sigma = dt/dx^4 with dt = 1e-6, dx = 1/1024, 100 implicit time steps per
benchmark step.  One benchmark step is the whole path on one batch already
resident in device memory: hyperdiffusion_factor (build the operator, factor
it once with the periodic-reduction quantities) then hyperdiffusion_solve
(all 100 solves -- forward sweep, corner/interface solve, backward sweep --
on every system); together they are exactly hyperdiffusion_step.

Timing protocol: W untimed warm-up steps, then exactly K timed steps (50 by
default)
bracketed by torch.cuda.synchronize(); `value` is the whole-job throughput
(unknowns of the K steps over the wall time).  Every call is also bracketed
by HIP events on the stream the library launches on, giving per-call medians
with p10 / p90 (`timing`); for the headline the event pair around
hyperdiffusion_solve times the register-resident step kernel alone (one
launch), which is what the roofline uses.  After the timed region the same
call is made on the initial state and a sample of systems is compared with
the oracle (`parity`).

Output: ONE JSON line (metric, value = unknowns solved per second, ...),
with "timing", "parity", a "roofline" object for the dominant kernel (the
headline's is bound by fp64 vector arithmetic: 17 algorithmic flops per
unknown per time step against the 78.6 TFLOP/s fp64 vector peak; its "hbm"
part gives the state's algorithmic bytes per launch and the measured
counter bytes over the kernel time) and a "cpu_baseline" object (the
oracle, built with gcc -O3 -march=native -fopenmp on this host, timed on a
bounded sample of the same workload with all of this host's cores and with
one thread, median of 5 runs each, CPU model and core counts stated).

    python bench.py [--steps K] [--warmup W] [--workload {0,...,14}]

--workload selects another workload for manual measurements
(0: the small periodic case, N = 256, 64 systems, 10 steps from seeded Fourier
modes -- latency-bound, reported for completeness; 2: general pentadiagonal 512 x 65536 factor+solve, --dtype f64|f32; 3: Hines mono
512 x 100000; 4: Hines multi, 32768 neurons of 256..2048 compartments,
20 solves per step; 5: the default shape time-stepped with Crank-Nicolson,
theta = 1/2, 24 algorithmic flops per unknown per time step; 6: the same grid
and batch for the Cahn-Hilliard equation, semi-implicit, 25 flops; 7, 8:
batched tridiagonal solves, 512 x 256000 and 8192 x 20000, --dtype f64|f32;
9: periodic pentadiagonal 512 x 65536 with per-system coefficients, fused
factor+solve, --dtype f64|f32; 10: Hines mono 512 x 256, a batch too small
for one lane per neuron, solved with the per-level section schedule; 11, 12:
workloads 3 and 4 with their trees numbered depth first, parents arbitrarily
far back; 13: Hines mono, one tree of 960 compartments x 53328 neurons, the
thirty-two-lane separator schedule; 14: Hines mono, one tree of 2000
compartments numbered depth first x 25600 neurons, the sixty-four-lane
separator schedule).
HBM-bound workloads also report the measured bandwidth of a plain 1 GiB
device copy (copy_gbs) and the kernel's fraction of it (frac_of_copy): a
stream that writes cannot exceed it.  Only one GPU is used; --gpus above 1
exits.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
FP64_VALU_PEAK_TFLOPS = 78.6   # MI355X fp64 vector peak (256 CUs x 128 flop/clk x 2.4 GHz)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _stats(xs):
    """Median, 10th and 90th percentile of a list of times (ms)."""
    import numpy as np
    a = np.asarray(xs, dtype=float)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def _time_steps(segments, steps, warmup):
    """Warm up, then time exactly `steps` steps bracketed by synchronisation.

    A step runs the callables in `segments` in order; HIP events on the
    current stream (the one the library launches on) are recorded before the
    first and after each, so that every segment of every step is timed on
    the device.  Returns the wall time of the timed steps and, per segment,
    the list of its per-step times in ms."""
    import torch
    for _ in range(warmup):
        for f in segments:
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(segments) + 1)]
           for _ in range(steps)]
    t0 = time.perf_counter()
    for ev in evs:
        ev[0].record()
        for k, f in enumerate(segments):
            f()
            ev[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [[ev[k].elapsed_time(ev[k + 1]) for ev in evs] for k in range(len(segments))]
    return wall, per


def _time_loop(fn, steps, warmup):
    """One-segment _time_steps: (wall, per-step ms)."""
    wall, per = _time_steps([fn], steps, warmup)
    return wall, per[0]


def _resident_kernel(n, batch, ex):
    """Name of the resident step kernel the library launches for (n, batch):
    16-row chunks for n = 256 up to 16384 systems, 16 chunks for n = 384 ..
    896 in steps of 128, 64-row chunks otherwise."""
    if n == 256 and batch <= 16384:
        return f"k_hyper_resident<16,16,{ex}>"
    if n in (384, 512, 640, 768, 896):
        return f"k_hyper_resident<{n // 16},16,{ex}>"
    return f"k_hyper_resident<64,{n // 64},{ex}>"


def _source_hash(relpath):
    """Hash of a kernel source's code: comments and blank lines do not count
    (the sources hold no comment markers inside string literals)."""
    import hashlib
    import re
    with open(os.path.join(ROOT, relpath), encoding="utf-8") as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def _traffic(key):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel's source changed after the counters were taken."""
    try:
        with open(PROFILE_TRAFFIC) as fh:
            ent = json.load(fh).get(key)
    except (OSError, ValueError):
        return None
    if not ent or ent.get("source_sha256") != _source_hash(ent["source"]):
        return None
    return ent["bytes_per_launch"]


def pmc_summary(args):
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE CSVs into a traffic entry.

    Each counter is scaled by what it reads for a plain 1 GiB device copy
    (bench.py --calibrate-copy) so that the copy counts exactly 1 GiB read and
    1 GiB written; the entry is keyed by --pmc-key and tied to a hash of the
    kernel's source file."""
    import csv
    fetch, write, cfetch, cwrite = args.pmc_summary

    def mean_of(path, match):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if match in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no dispatch of {match!r} in {path}")
        return sum(vals) / len(vals), len(vals)

    gib_kib = float(1 << 20)
    f_copy, _ = mean_of(cfetch, args.copy_match)
    w_copy, _ = mean_of(cwrite, args.copy_match)
    f_scale, w_scale = gib_kib / f_copy, gib_kib / w_copy
    if args.pmc_calls_match:
        # a call of several kernels: all matching dispatches summed, divided
        # by the number of calls (dispatches of the one kernel named here)
        def per_call(path):
            rows = list(csv.DictReader(open(path)))
            tot = sum(float(r["Counter_Value"]) for r in rows if args.pmc_match in r["Kernel_Name"])
            calls = sum(1 for r in rows if args.pmc_calls_match in r["Kernel_Name"])
            if not calls:
                raise SystemExit(f"no dispatch of {args.pmc_calls_match!r} in {path}")
            return tot / calls, calls
        f_k, nf = per_call(fetch)
        w_k, nw = per_call(write)
    else:
        f_k, nf = mean_of(fetch, args.pmc_match)
        w_k, nw = mean_of(write, args.pmc_match)
    fb, wb = f_k * f_scale * 1024, w_k * w_scale * 1024
    ent = {"kernel": args.pmc_match, "bytes_per_launch": fb + wb, "fetch_bytes": fb,
           "write_bytes": wb, "fetch_scale": f_scale, "write_scale": w_scale,
           "dispatches": [nf, nw], "source": args.pmc_source,
           "source_sha256": _source_hash(args.pmc_source)}
    try:
        with open(PROFILE_TRAFFIC) as fh:
            allt = json.load(fh)
    except (OSError, ValueError):
        allt = {}
    allt[args.pmc_key] = ent
    with open(PROFILE_TRAFFIC, "w") as fh:
        json.dump(allt, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({args.pmc_key: ent}), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(run_sample, unknowns_per_system, label, seconds):
    """The oracle as it stands, timed on this host: built here with gcc -O3
    -march=native -fopenmp (oracle.TIMING_CFLAGS), run on a sample of the
    workload sized so that one run takes about seconds / 12, five runs with
    all the threads OpenMP gives it and five with one thread, medians
    reported (about `seconds` of CPU work in all)."""
    import tempfile
    import oracle
    oracle.use_library(oracle.build_timing(tempfile.mkdtemp(prefix="orc_timing_")))
    legs = {}
    for key, req in (("all", 0), ("one", 1)):
        used = oracle.set_threads(req)
        k, t = 4, 0.0
        while True:
            t0 = time.perf_counter()
            run_sample(k)
            t = time.perf_counter() - t0
            if t >= seconds / 40 or k >= 1 << 20:
                break
            k = int(k * min(16.0, max(2.0, seconds / 40 / max(t, 1e-4))))
        k = max(1, int(k * seconds / 12 / max(t, 1e-6)))
        runs = []
        for _ in range(5):
            t0 = time.perf_counter()
            run_sample(k)
            runs.append(time.perf_counter() - t0)
        med = statistics.median(runs)
        legs[key] = {"value": k * unknowns_per_system / med, "systems_per_s": k / med,
                     "threads": used, "sample": f"{k} {label}", "runs_s": [round(r, 3) for r in runs]}
    a = legs["all"]
    return {"value": a["value"], "unit": "unknowns/s", "cores": a["threads"], "kind": "oracle",
            "sample": f"{a['sample']}, median of 5 runs of {statistics.median(a['runs_s']):.2f} s",
            "systems_per_s": a["systems_per_s"],
            "one_thread": {"value": legs["one"]["value"], "systems_per_s": legs["one"]["systems_per_s"],
                           "sample": f"{legs['one']['sample']}, median of 5 runs",
                           "runs_s": legs["one"]["runs_s"]},
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)),
            "build": "gcc " + " ".join(oracle.TIMING_CFLAGS)}


def _max_col_err(got, ref, scale=None):
    """Largest per-system normwise relative error of (n, k) arrays."""
    import numpy as np
    den = np.linalg.norm(ref if scale is None else scale, axis=0)
    return float(np.max(np.linalg.norm(got - ref, axis=0) / den))


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def bench_hyperdiffusion(args, which=1):
    """Workloads 1 (implicit), 5 (Crank-Nicolson) and 6 (Cahn-Hilliard): the
    register-resident periodic solver with the matching right-hand side."""
    import numpy as np
    import torch
    import banded_pde_solvers_amd as bps
    import workloads as W

    cfg = W.WORKLOADS[which]
    kind = cfg["kind"]
    n, batch, nsteps, dt, dx = cfg["n"], cfg["batch"], cfg["nsteps"], cfg["dt"], cfg["dx"]
    theta = cfg.get("theta")
    dev = "cuda:0"
    if kind == "cahn_hilliard":
        C0 = torch.as_tensor(W.cahn_hilliard_quench(n, batch), device=dev)
    elif which == 0:
        C0 = torch.as_tensor(W.hyperdiffusion_modes(n, batch).C0, device=dev)
    else:
        C0 = torch.as_tensor(W.hyperdiffusion_random(n, batch), device=dev)
    C = C0.clone()
    if kind == "hyperdiffusion":
        # the headline: factor once, then the 100 steps (one kernel launch)
        work = torch.empty(bps.hyperdiffusion_work_bytes(n, batch), dtype=torch.uint8, device=dev)
        segs = [lambda: bps.hyperdiffusion_factor(n, dt, dx, work),
                lambda: bps.hyperdiffusion_solve(C, dt, dx, nsteps, work)]
        run = lambda: [f() for f in segs]
    elif kind == "hyperdiffusion_theta":
        work = torch.empty(bps.hyperdiffusion_theta_work_bytes(n, batch), dtype=torch.uint8, device=dev)
        run = lambda: bps.hyperdiffusion_theta_step(C, dt, dx, theta, nsteps, work)
        segs = [run]
    else:
        gamma, mob = cfg["gamma"], cfg["mobility"]
        work = torch.empty(bps.cahn_hilliard_work_bytes(n, batch), dtype=torch.uint8, device=dev)
        run = lambda: bps.cahn_hilliard_step(C, dt, dx, gamma, mob, theta, nsteps, work)
        segs = [run]
    wall, per = _time_steps(segs, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    call = [sum(x) for x in zip(*per)]
    kern = per[-1]            # the step kernel alone (headline), else the whole call
    unknowns = n * batch * nsteps
    # The solve keeps every system in registers for all time steps, so HBM
    # sees the state once in and once out per call: the kernel is bound by
    # fp64 vector arithmetic.  Algorithmic flops per unknown per time step of
    # the periodic LU solve: forward 2 FMA + 1 MUL, corner dot products 2 FMA,
    # back substitution 2 FMA, rank-2 corner correction 2 FMA = 17 flops.
    # A theta < 1 right-hand side adds the explicit stencil, at least 7 flops
    # in its symmetric form e0 x_i + e1 (x_i-1 + x_i+1) + e2 (x_i-2 + x_i+2);
    # the Cahn-Hilliard term r (phi_i-1 - 2 phi_i + phi_i+1), phi = x^3 - x
    # (x (x x - 1): 3 flops per row), adds 3 + 3 + 2 = 8.
    flops_per = 17.0
    if theta is not None and theta != 1.0:
        flops_per += 7.0
    if kind == "cahn_hilliard":
        flops_per += 8.0
    kern_ms = _stats(kern)["median"]
    alg_flops = flops_per * unknowns
    achieved = alg_flops / (kern_ms * 1e-3) / 1e12
    hbm_bytes = 16.0 * n * batch                     # C read once, written once
    # counter traffic was taken on the N = 1024 x 16384 workloads only
    traffic = _traffic({"hyperdiffusion": "hyperdiffusion", "hyperdiffusion_theta": "hyperdiffusion_theta",
                        "cahn_hilliard": "cahn_hilliard"}[kind]) if which in (1, 5, 6) else None
    label = {"hyperdiffusion": "periodic hyperdiffusion implicit steps",
             "hyperdiffusion_theta": "periodic hyperdiffusion Crank-Nicolson steps",
             "cahn_hilliard": "periodic Cahn-Hilliard semi-implicit steps"}[kind]
    config = {"workload": cfg["name"], "n": n, "batch": batch, "time_steps_per_step": nsteps,
              "dt": dt, "dx": dx}
    if kind == "cahn_hilliard":
        r = cfg["mobility"] * dt / dx ** 2
        config.update(gamma=cfg["gamma"], mobility=cfg["mobility"], theta=theta, r=r,
                      sigma=cfg["gamma"] * r / dx ** 2)
    else:
        config.update(sigma=dt / dx ** 4, scheme="implicit" if theta is None else f"theta = {theta}")
    config["coefficients"] = "constant (factor once)"
    timing = {"call_ms": _stats(call), "systems_per_s": batch * args.steps / wall,
              "time_steps_per_s": nsteps * args.steps / wall}
    if kind == "hyperdiffusion":
        timing["factor_ms"] = _stats(per[0])
        timing["solve_kernel_ms"] = _stats(kern)
        timed = f"{_resident_kernel(n, batch, 0)} alone (HIP events around hyperdiffusion_solve)"
    else:
        timed = "whole call (set-up kernel included)"
    line = {
        "metric": "unknowns solved/s (fp64), " + label,
        "value": unknowns * args.steps / wall,
        "unit": "unknowns/s",
        "ms_per_step": ms_step,
        "dtype": "f64",
        "config": config,
        "timing": timing,
        "roofline": {"bound": "alu", "kernel": _resident_kernel(n, batch, {"hyperdiffusion": 0,
                     "hyperdiffusion_theta": 1, "cahn_hilliard": 2}[kind]),
                     "achieved": achieved, "peak": FP64_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP64_VALU_PEAK_TFLOPS, "traffic": traffic,
                     "kernel_ms": kern_ms, "timed": timed,
                     "flops_per_unknown_step": flops_per, "flops_per_launch": alg_flops,
                     "hbm": {"algorithmic_bytes_per_launch": hbm_bytes,
                             "counter_bytes_per_launch": traffic,
                             "achieved_gbs": None if traffic is None else traffic / (kern_ms * 1e-3) / 1e9,
                             "frac_of_peak": None if traffic is None else
                             traffic / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                     "model_gbs_if_state_streamed_every_step":
                         16.0 * unknowns / (kern_ms * 1e-3) / 1e9},
    }
    # parity on a sample of systems, outside the timed region: the call on
    # the initial state against the oracle's trajectory (R12: relative to
    # the norm of C0, <= 2e-9 after 100 steps)
    import oracle
    cols = np.unique(np.r_[0, batch - 1, np.random.default_rng(11).integers(0, batch, 14)])
    C.copy_(C0)
    run()
    torch.cuda.synchronize()
    got = C[:, cols].cpu().numpy()
    c0 = C0[:, cols].cpu().numpy()
    if kind == "hyperdiffusion":
        ref = oracle.hyperdiffusion(W.to_flat(c0), dt, dx, nsteps).T
    elif kind == "hyperdiffusion_theta":
        ref = oracle.hyperdiffusion_theta(W.to_flat(c0), dt, dx, theta, nsteps).T
    else:
        ref = oracle.cahn_hilliard(W.to_flat(c0), dt, dx, cfg["gamma"], cfg["mobility"], theta, nsteps).T
    par = {"systems_checked": int(len(cols)),
           "max_rel_err_vs_oracle": _max_col_err(got, ref, scale=c0),
           "norm": "||C_gpu - C_oracle|| / ||C0|| per system, after the call's "
                   f"{nsteps} steps"}
    if kind == "hyperdiffusion":
        # one implicit step (one solve per system) with the same factors: the
        # per-solve error, relative to the oracle's solution
        C.copy_(C0)
        bps.hyperdiffusion_solve(C, dt, dx, 1, work)
        torch.cuda.synchronize()
        ref1 = oracle.hyperdiffusion(W.to_flat(c0), dt, dx, 1).T
        par["per_solve_max_rel_err_vs_oracle"] = _max_col_err(C[:, cols].cpu().numpy(), ref1)
        par["per_solve_norm"] = "||x_gpu - x_oracle|| / ||x_oracle|| per system, one step"
    line["parity"] = par
    if not args.no_cpu_baseline:
        if kind == "cahn_hilliard":
            Cs = W.cahn_hilliard_quench(n, 2048, rng=np.random.default_rng(77))
        else:
            Cs = W.hyperdiffusion_random(n, 2048, rng=np.random.default_rng(77))

        def sample(k):
            reps = (k + 2047) // 2048
            for r in range(reps):
                kk = min(2048, k - r * 2048)
                x = W.to_flat(Cs[:, :kk])
                if kind == "hyperdiffusion":
                    oracle.hyperdiffusion(x, dt, dx, nsteps)
                elif kind == "hyperdiffusion_theta":
                    oracle.hyperdiffusion_theta(x, dt, dx, theta, nsteps)
                else:
                    oracle.cahn_hilliard(x, dt, dx, cfg["gamma"], cfg["mobility"], theta, nsteps)
        line["cpu_baseline"] = _cpu_baseline(sample, n * nsteps, f"systems x {nsteps} steps",
                                             args.cpu_seconds)
    return line


def bench_penta(args, which=2):
    """Workloads 2 (non-periodic) and 9 (periodic): fused factor + solve of
    pentadiagonal systems with per-system coefficients."""
    import numpy as np
    import torch
    import banded_pde_solvers_amd as bps
    import workloads as W

    cfg = W.WORKLOADS[which]
    cyclic = cfg["kind"] == "penta_cyclic"
    n, batch = cfg["n"], cfg["batch"]
    dt = torch.float32 if args.dtype == "f32" else torch.float64
    pb = W.penta_dominant(n, batch, cyclic=cyclic, rng=W.rng_for(which))
    cols = np.unique(np.r_[0, batch - 1, np.random.default_rng(12).integers(0, batch, 62)])
    sample_in = [v[:, cols].copy() for v in (*pb.diagonals, pb.f)]
    dg = [torch.as_tensor(v, device="cuda:0").to(dt) for v in pb.diagonals]
    f0 = torch.as_tensor(pb.f, device="cuda:0").to(dt)
    x = f0.clone()
    code = bps.BPS_F32 if dt == torch.float32 else bps.BPS_F64
    work = torch.empty(bps.bps_penta_work_bytes(n, batch, batch, code, cyclic=cyclic),
                       dtype=torch.uint8, device="cuda:0")
    del pb

    if args.split:
        # the page's two calls: factor (the factors of every system written
        # out), then solve with them
        fac = torch.empty(bps.bps_penta_factor_bytes(n, batch, batch, code,
                                                     bps.BPS_CYCLIC if cyclic else 0),
                          dtype=torch.uint8, device="cuda:0")
        solve = bps.penta_cyclic_solve_batch if cyclic else bps.penta_solve_batch

        def step():
            bps.penta_factor_batch(*dg, fac, cyclic=cyclic)
            solve(fac, x)
    else:
        def step():
            bps.penta_factor_solve_batch(*dg, x, work, cyclic=cyclic)
    wall, per = _time_loop(step, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    if args.split:
        kname = "k_penta_factor + " + ("k_penta_cyclic_solve" if cyclic else "k_penta_solve")
    elif n % 16 == 0 and 2 <= n // 16 <= 64 and (not cyclic or (n // 16) & (n // 16 - 1) == 0):
        kname = "k_penta_spike"
    else:
        kname = "k_penta_fused"
    es = 4 if dt == torch.float32 else 8
    unknowns = n * batch
    alg_bytes = 7.0 * es * unknowns                  # 5 diagonals + f in, x out
    kern_ms = _stats(per)["median"]
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    traffic = None if args.split else _traffic(kname[2:] + ("_cyclic_" if cyclic else "_") + args.dtype)
    line = {
        "metric": f"unknowns solved/s ({args.dtype}), " +
                  ("periodic" if cyclic else "general") + " pentadiagonal factor+solve",
        "value": unknowns * args.steps / wall, "unit": "unknowns/s", "ms_per_step": ms_step,
        "dtype": args.dtype,
        "config": {"workload": cfg["name"], "n": n, "batch": batch, "coefficients": "per system",
                   "periodic": cyclic, "calls": "factor, then solve" if args.split else "fused"},
        "timing": {"call_ms": _stats(per), "systems_per_s": batch * args.steps / wall},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel_ms": kern_ms,
                     "timed": "whole call" + (" (the chunked kernel, then the masked second pass)"
                                              if cyclic and not args.split else ""),
                     "bytes_per_launch": alg_bytes,
                     "counter_gbs": None if traffic is None else traffic / (kern_ms * 1e-3) / 1e9},
    }
    import oracle
    x.copy_(f0)
    step()
    torch.cuda.synchronize()
    got = x[:, cols].cpu().double().numpy()
    rin = [v.astype(np.float32).astype(np.float64) if es == 4 else v for v in sample_in]
    ref, _ = oracle.penta_solve(*(W.to_flat(v) for v in rin), cyclic=cyclic)
    line["parity"] = {"systems_checked": int(len(cols)),
                      "max_rel_err_vs_oracle": _max_col_err(got, W.to_interleaved(ref)),
                      "norm": "||x_gpu - x_oracle|| / ||x_oracle|| per system (fp32: the fp64 "
                              "oracle of the fp32-rounded inputs)"}
    if not args.no_cpu_baseline:
        small = W.penta_dominant(n, 4096, cyclic=cyclic, rng=np.random.default_rng(5))
        fl = [W.to_flat(v) for v in (*small.diagonals, small.f)]

        def sample(k):
            for r in range((k + 4095) // 4096):
                kk = min(4096, k - r * 4096)
                oracle.penta_solve(*(v[:kk] for v in fl), cyclic=cyclic)
        line["cpu_baseline"] = _cpu_baseline(sample, n, "systems", args.cpu_seconds)
    return line


def bench_tri(args, which):
    """Workloads 7, 8: batched tridiagonal solves (the Hines page's
    cuThomasBatch test cases), per-system coefficients, fp64 or fp32."""
    import numpy as np
    import torch
    import banded_pde_solvers_amd as bps
    import workloads as W

    cfg = W.WORKLOADS[which]
    n, batch = cfg["n"], cfg["batch"]
    dt = torch.float32 if args.dtype == "f32" else torch.float64
    tb = W.tri_dominant(n, batch)
    cols = np.unique(np.r_[0, batch - 1, np.random.default_rng(13).integers(0, batch, 62)])
    sample_in = [v[:, cols].copy() for v in (tb.a, tb.b, tb.c, tb.y)]
    a, b, c, y = (torch.as_tensor(v, device="cuda:0").to(dt) for v in (tb.a, tb.b, tb.c, tb.y))
    y0 = y.clone()
    del tb
    code = bps.BPS_F32 if dt == torch.float32 else bps.BPS_F64
    work = torch.empty(bps.tri_work_bytes(n, batch, code), dtype=torch.uint8, device="cuda:0")

    def step():
        bps.tri_solve_batch(a, b, c, y, work)
    wall, per = _time_loop(step, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    if n % 16 == 0 and 2 <= n // 16 <= 64:
        kname = "k_tri_chunk"
    elif n % 16 == 0 and 64 < n // 16 <= 65535:
        kname = "k_tri_part"        # five kernels per call: timed as a whole
    else:
        kname = "k_tri_thomas"
    es = 4 if dt == torch.float32 else 8
    unknowns = n * batch
    alg_bytes = 5.0 * es * unknowns                  # a, b, c, y in, u out
    kern_ms = _stats(per)["median"]
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    traffic = _traffic(f"{kname[2:]}_n{n}_{args.dtype}")
    line = {
        "metric": f"unknowns solved/s ({args.dtype}), batched tridiagonal solve",
        "value": unknowns * args.steps / wall, "unit": "unknowns/s", "ms_per_step": ms_step,
        "dtype": args.dtype,
        "config": {"workload": cfg["name"], "n": n, "batch": batch, "coefficients": "per system"},
        "timing": {"call_ms": _stats(per), "systems_per_s": batch * args.steps / wall},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel_ms": kern_ms, "timed": "whole call",
                     "bytes_per_launch": alg_bytes,
                     "counter_gbs": None if traffic is None else traffic / (kern_ms * 1e-3) / 1e9},
    }
    import oracle
    y.copy_(y0)
    step()
    torch.cuda.synchronize()
    got = y[:, cols].cpu().double().numpy()
    rin = [v.astype(np.float32).astype(np.float64) if es == 4 else v for v in sample_in]
    ref, _ = oracle.thomas_solve(*(W.to_flat(v) for v in rin))
    line["parity"] = {"systems_checked": int(len(cols)),
                      "max_rel_err_vs_oracle": _max_col_err(got, W.to_interleaved(ref)),
                      "norm": "||u_gpu - u_oracle|| / ||u_oracle|| per system"}
    if not args.no_cpu_baseline:
        k0 = max(1, min(batch, (1 << 22) // n))
        small = W.tri_dominant(n, k0, rng=np.random.default_rng(9))
        fl = [W.to_flat(v) for v in (small.a, small.b, small.c, small.y)]

        def sample(k):
            for r in range((k + k0 - 1) // k0):
                kk = min(k0, k - r * k0)
                oracle.thomas_solve(*(v[:kk] for v in fl))
        line["cpu_baseline"] = _cpu_baseline(sample, n, "systems", args.cpu_seconds)
    return line


def _hines_common(args, multi, which=None):
    import numpy as np
    import torch
    import banded_pde_solvers_amd as bps
    import workloads as W

    cfg = W.WORKLOADS[which if which is not None else (4 if multi else 3)]
    sched = {"auto": bps.BPS_HINES_AUTO, "lanes": bps.BPS_HINES_LANES, "split": bps.BPS_HINES_SPLIT,
             "levels": bps.BPS_HINES_LEVELS, "sep": bps.BPS_HINES_SEP}[args.hines_schedule]
    if multi:
        mm = W.hines_multi(cfg["batch"], cfg["nmin"], cfg["nmax"],
                           rng=W.rng_for(which) if which is not None else None, dfs=cfg.get("dfs", False))
        plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False, schedule=sched)
        arrs = []
        for v in (mm.u, mm.l, mm.d, mm.rhs):
            t = torch.empty(plan.elems, dtype=torch.float64, device="cuda:0")
            bps.hines_pack(plan, torch.as_tensor(v, device="cuda:0"), t)
            arrs.append(t)
        nsolve = cfg["nsteps"]
        stats = {"mean_n": float(mm.sizes.mean()), "padded_elems": plan.elems,
                 "trees_on_two_lanes": plan.split}
    else:
        hm = W.hines_mono(cfg["n"], cfg["batch"], rng=W.rng_for(which if which is not None else 3),
                          dfs=cfg.get("dfs", False))
        plan = bps.hines_plan_create(cfg["batch"], [cfg["n"]], hm.parent, mono=True, schedule=sched)
        arrs = [torch.as_tensor(v, device="cuda:0") for v in (hm.u, hm.l, hm.d, hm.rhs)]
        nsolve = 1
        stats = W.tree_stats(hm.parent)
    u, l, d, rhs = arrs
    r0 = rhs.clone()
    work = torch.empty(bps.hines_work_bytes(plan), dtype=torch.uint8, device="cuda:0")

    # one step: nsolve solves, rhs_{k+1} = V_k, d restored (kept constant);
    # each solve is one segment, timed by its own events
    solve = lambda: bps.hines_solve_batch(plan, u, l, d, rhs, work)
    wall, per = _time_steps([solve] * nsolve, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    per_solve = [t for seg in per for t in seg]
    unknowns = plan.unknowns * nsolve
    per_unknown = 44.0 if multi else 40.0            # u, l, d, rhs in, V out (+ parent)
    kern_ms = _stats(per_solve)["median"]
    alg_bytes = per_unknown * plan.unknowns
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    if multi:
        loc = np.arange(len(mm.parent)) - np.repeat(mm.offsets[:-1], mm.sizes)
        maxd = int(np.max(np.where(loc > 0, loc - mm.parent, 0)))
    else:
        maxd = int(stats["max_parent_distance"])
    general = not plan.uses_levels and not plan.uses_sep and maxd > 16      # beyond the 16-slot ring
    kname = ("k_hines_levels" if plan.uses_levels else
             "k_hines<general>" if general else
             ("k_hines_sepm" if plan.uses_sep else "k_hines_split" if plan.split else "k_hines_multi")
             if multi else "k_hines_sep" if plan.uses_sep else "k_hines_mono_reg")
    tkey = ("hines_levels" if plan.uses_levels else "hines_general" if general else
            ("hines_sepm" if plan.uses_sep else "hines_split" if plan.split else "hines_multi")
            if multi else
            f"hines_sep_n{cfg['n']}_b{cfg['batch']}" if plan.uses_sep else "hines_mono")
    traffic = _traffic(tkey + ("_dfs" if cfg.get("dfs") else ""))
    line = {
        "metric": "unknowns solved/s (fp64), Hines " + ("multi" if multi else "mono"),
        "value": unknowns * args.steps / wall, "unit": "unknowns/s", "ms_per_step": ms_step,
        "dtype": "f64",
        "config": {"workload": cfg["name"], "solves_per_step": nsolve, **stats},
        "timing": {"solve_ms": _stats(per_solve), "systems_per_s": plan.batch * nsolve * args.steps / wall},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "schedule": "levels" if plan.uses_levels else
                                 "two lanes for the largest trees" if plan.split else
                                 ("separators, every tree on its own lanes" if multi else
                                  f"{bps.hines_sep_schedule(hm.parent)['lanes']} lanes per neuron (separators)")
                                 if plan.uses_sep else
                                 "one lane per neuron, general variant (parents beyond 16)" if general else
                                 "one lane per neuron",
                     "kernel_ms": kern_ms, "timed": "one solve call", "bytes_per_launch": alg_bytes,
                     "counter_gbs": None if traffic is None else traffic / (kern_ms * 1e-3) / 1e9},
    }
    import oracle
    rhs.copy_(r0)
    solve()
    torch.cuda.synchronize()
    errs = []
    if multi:
        flat = torch.empty(plan.unknowns, dtype=torch.float64, device="cuda:0")
        bps.hines_unpack(plan, rhs, flat)
        out = flat.cpu().numpy()
        pick = np.unique(np.r_[0, mm.batch - 1, np.random.default_rng(14).integers(0, mm.batch, 30)])
        for s_ in pick:
            p_, u_, l_, d_, r_ = mm.neuron(s_)
            V, _ = oracle.hines_solve(p_, u_, l_, d_, r_)
            got = out[mm.offsets[s_]:mm.offsets[s_ + 1]]
            errs.append(np.linalg.norm(got - V[0]) / np.linalg.norm(V[0]))
    else:
        cols = np.unique(np.r_[0, cfg["batch"] - 1,
                               np.random.default_rng(14).integers(0, cfg["batch"], 62)])
        got = rhs[:, cols].cpu().numpy()
        V, _ = oracle.hines_solve(hm.parent, *(W.to_flat(v[:, cols]) for v in (hm.u, hm.l, hm.d, hm.rhs)))
        errs.append(_max_col_err(got, W.to_interleaved(V)))
        pick = cols
    line["parity"] = {"systems_checked": int(len(pick)), "max_rel_err_vs_oracle": float(max(errs)),
                      "norm": "||V_gpu - V_oracle|| / ||V_oracle|| per neuron, one solve"}
    if not args.no_cpu_baseline:
        if multi:
            small = W.hines_multi(2048, cfg["nmin"], cfg["nmax"], rng=np.random.default_rng(9),
                                  dfs=cfg.get("dfs", False))

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
            small = W.hines_mono(cfg["n"], 4096, rng=np.random.default_rng(9), dfs=cfg.get("dfs", False))
            fl = [W.to_flat(v) for v in (small.u, small.l, small.d, small.rhs)]

            def sample(k):
                for r in range((k + 4095) // 4096):
                    kk = min(4096, k - r * 4096)
                    oracle.hines_solve(small.parent, *(v[:kk] for v in fl))
            line["cpu_baseline"] = _cpu_baseline(sample, cfg["n"], "neurons", args.cpu_seconds)
    plan.close()
    return line


def _copy_gbs():
    """Measured device-copy bandwidth (1 GiB read + 1 GiB written, median of
    5): the practical ceiling of a stream that writes, beside the 8 TB/s
    peak."""
    import torch
    nbytes = 1 << 30
    src = torch.ones(nbytes // 8, dtype=torch.float64, device="cuda:0")
    dst = torch.empty_like(src)
    _, per = _time_loop(lambda: dst.copy_(src), 5, 2)
    del src, dst
    return 2 * nbytes / (statistics.median(per) * 1e-3) / 1e9


def calibrate_copy(args):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    nbytes = 1 << 30
    src = torch.ones(nbytes // 8, dtype=torch.float64, device="cuda:0")
    dst = torch.empty_like(src)
    wall, per = _time_loop(lambda: dst.copy_(src), args.steps, args.warmup)
    ms = statistics.mean(per)
    print(json.dumps({"calibration": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "ms": ms, "GBs": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # median of 50 timed calls (the SpEC page's benchmarking section)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1, choices=list(range(0, 15)))
    ap.add_argument("--dtype", default="f64", choices=["f64", "f32"], help="workloads 2, 7, 8, 9")
    ap.add_argument("--split", action="store_true",
                    help="workloads 2, 9: time the separate factor and solve calls instead")
    ap.add_argument("--hines-schedule", default="auto", choices=["auto", "lanes", "split", "levels", "sep"],
                    help="workloads 3, 4, 10-14: the plan's schedule (BPS_HINES_*)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPYFETCH", "COPYWRITE"),
                    help="write profiles/traffic.json from rocprofv3 counter CSVs and exit")
    ap.add_argument("--pmc-key", default="hyperdiffusion")
    ap.add_argument("--pmc-match", default="k_hyper_resident<")
    ap.add_argument("--pmc-source", default="banded_pde_solvers_amd/csrc/hyper.hip")
    ap.add_argument("--copy-match", default="copyBuffer")
    ap.add_argument("--pmc-calls-match", default=None,
                    help="sum the --pmc-match dispatches per call of this kernel")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: the systems of a batch are independent, "
                  "so a multi-GPU run would split the batch by columns and add nothing to "
                  "measure per GPU; rerun with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args)
        return
    import banded_pde_solvers_amd as bps
    bps.load_library()
    fn = {0: lambda a: bench_hyperdiffusion(a, 0), 1: bench_hyperdiffusion, 2: bench_penta, 3: lambda a: _hines_common(a, False),
          4: lambda a: _hines_common(a, True), 5: lambda a: bench_hyperdiffusion(a, 5),
          6: lambda a: bench_hyperdiffusion(a, 6), 7: lambda a: bench_tri(a, 7),
          8: lambda a: bench_tri(a, 8), 9: lambda a: bench_penta(a, 9),
          10: lambda a: _hines_common(a, False, 10), 11: lambda a: _hines_common(a, False, 11),
          12: lambda a: _hines_common(a, True, 12), 13: lambda a: _hines_common(a, False, 13),
          14: lambda a: _hines_common(a, False, 14)}[args.workload]
    line = fn(args)
    roof = line.get("roofline")
    if roof and roof.get("bound") == "hbm":
        roof["copy_gbs"] = _copy_gbs()
        roof["frac_of_copy"] = roof["achieved"] / roof["copy_gbs"]
    out = {"metric": line.pop("metric"), "value": line.pop("value"), "unit": line.pop("unit"),
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": line.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": line.pop("dtype"), "data": "synthetic (seeded)",
           "config": line.pop("config")}
    out.update(line)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
