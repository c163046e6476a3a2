"""Benchmark: PCG ms/solve and M-apply+SpMV bandwidth against the HBM roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N8k]

A step is one complete H-matrix-preconditioned PCG solve (init, apply, SpMV,
updates and fp64 reductions until ||r|| <= 1e-6 ||b||) of the named workload,
with A, the factors and b already resident in device memory.  The default
workload is the N = 8,192 system (3D 7-point variable-coefficient Poisson on a
16 x 16 x 32 Morton-ordered grid, K = 64 leaves, 6 tile levels).

Printed: one JSON line on stdout.  `value` is ms per solve (lower is better).
`roofline` covers the M-apply + SpMV pair, timed per call with HIP events on
the library's stream, against MI355X's 8 TB/s HBM peak, using algorithmic bytes
(each factor, matrix entry and vector read or written once per call).
`cpu_baseline` times the fp64 numpy oracle on a bounded sample on host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "PCG ms/solve and M-apply+SpMV HBM GB/s (fraction of peak) at N=8,192"


def apply_bytes(n: int, K: int, levels: int, B: int = 1) -> int:
    """Algorithmic bytes of one M-apply: leaf factors, level slabs, gate, r in, y out."""
    L, R = 128, 32
    return B * 4 * (n * L + n * R * levels + n) + B * 8 * n


def spmv_bytes(n: int, nnz: int, B: int = 1) -> int:
    """Algorithmic bytes of one SpMV: values + column indices, row pointers, x in, y out."""
    return 8 * nnz + 4 * (B * n + 1) + 8 * B * n


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_solves(solver, b, tol, maxit, steps, warmup, torch):
    for _ in range(warmup):
        solver.solve(b, tol=tol, maxit=maxit)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    iters = None
    for _ in range(steps):
        res = solver.solve(b, tol=tol, maxit=maxit)
        iters = res.iterations
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, iters, res


def time_calls(fn, reps, torch):
    """Average duration of fn() with a HIP event pair around every call."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    for a, e in evs:
        a.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(e) for a, e in evs]
    return float(np.mean(ms)) * 1e3, float(np.median(ms)) * 1e3   # microseconds


def time_back_to_back(fn, reps, torch):
    stream = torch.cuda.current_stream()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    e.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(e) * 1e3 / reps


def cpu_baseline(batch, budget_s=12.0):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    sy = batch.system(0)
    t0 = time.perf_counter()
    solves = 0
    while True:
        oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), batch.tol, batch.maxit)
        solves += 1
        if time.perf_counter() - t0 > budget_s or solves >= 20:
            break
    ms = (time.perf_counter() - t0) * 1e3 / solves
    return {"value": round(ms, 3), "unit": "ms/solve", "cores": int(threads), "kind": "oracle",
            "sample": f"{solves} complete fp64 solves of the {batch.name} system (numpy oracle, "
                      f"{batch.n} unknowns)"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="N8k")
    ap.add_argument("--engine", type=int, default=0, help="0 auto, 1 graph, 2 persistent")
    ap.add_argument("--prec", type=int, default=0, help="0 fp64 vectors (default), 1 fp32 vectors")
    ap.add_argument("--no-variants", action="store_true", help="skip the engine/precision variants")
    ap.add_argument("--reps", type=int, default=300, help="calls per apply/SpMV timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-others", action="store_true", help="skip ms/solve of the other workloads")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this solver path is built and measured on a single "
              f"MI355X; --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2

    import torch

    from matrix_preconditioned_pcg_amd import hpcg
    from workloads import CONFIGS, make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)

    def run_config(name, steps, warmup, with_roofline, engine=None, prec=None):
        batch = make_config(name)
        solver = hpcg.Solver(batch.n, batch.row_ptr, batch.col, batch.val, batch=batch.batch,
                             levels=batch.levels)
        solver.set_factors(batch.U, batch.W, batch.g)
        engine = args.engine if engine is None else engine
        prec = args.prec if prec is None else prec
        if engine:
            solver.set_option(hpcg.HPCG_OPT_ENGINE, engine)
        solver.set_option(hpcg.HPCG_OPT_PRECISION, prec)
        b = torch.as_tensor(batch.b.reshape(-1)).cuda()
        ms, iters, res = time_solves(solver, b, batch.tol, batch.maxit, steps, warmup, torch)
        out = {"ms_per_solve": ms, "iterations": iters, "status": res.status,
               "engine": solver.last_engine, "batch": batch.batch, "n": batch.n}
        if with_roofline:
            r = torch.randn(batch.batch * batch.n, device="cuda", dtype=torch.float32)
            y = torch.empty_like(r)
            q = torch.empty_like(r)
            t_apply, t_apply_med = time_calls(lambda: hpcg.hpcg_apply_M(solver.handle, solver.part, r, y),
                                              args.reps, torch)
            t_spmv, t_spmv_med = time_calls(lambda: hpcg.hpcg_spmv(solver.handle, solver.part, r, q),
                                            args.reps, torch)

            def pair():
                hpcg.hpcg_spmv(solver.handle, solver.part, r, q)
                hpcg.hpcg_apply_M(solver.handle, solver.part, r, y)
            t_pair = time_back_to_back(pair, args.reps, torch)
            ab = apply_bytes(batch.n, batch.K, batch.levels, batch.batch)
            sb = spmv_bytes(batch.n, batch.nnz, batch.batch)
            out.update(apply_us=t_apply, apply_us_median=t_apply_med, spmv_us=t_spmv,
                       spmv_us_median=t_spmv_med, pair_back_to_back_us=t_pair,
                       apply_bytes=ab, spmv_bytes=sb)
        solver.close()
        return batch, out

    batch, main_out = run_config(args.config, args.steps, args.warmup, True)
    ab, sb = main_out["apply_bytes"], main_out["spmv_bytes"]
    t_sum = main_out["apply_us"] + main_out["spmv_us"]
    achieved = (ab + sb) / (t_sum * 1e-6) / 1e9
    others = {}
    if not args.no_others:
        for name in CONFIGS:
            if name == args.config:
                continue
            log(f"bench: {name}")
            _b, o = run_config(name, max(3, args.steps // 4), 1, False)
            others[name] = {"ms_per_solve": round(o["ms_per_solve"], 4), "iterations": o["iterations"]
                            if len(o["iterations"]) <= 4 else
                            {"min": min(o["iterations"]), "max": max(o["iterations"])},
                            "engine": o["engine"]}
    variants = {}
    if not args.no_variants:
        for label, eng, prec in (("persistent_vec64", 2, 0), ("persistent_vec32", 2, 1),
                                 ("graph_vec64", 1, 0), ("graph_vec32", 1, 1)):
            log(f"bench: variant {label}")
            _b, o = run_config(args.config, max(3, args.steps // 2), 1, False, eng, prec)
            variants[label] = {"ms_per_solve": round(o["ms_per_solve"], 4), "iterations": o["iterations"][0]}
    cpu = None if args.no_cpu else cpu_baseline(batch)
    iters = main_out["iterations"][0]
    line = {
        "metric": METRIC,
        "value": round(main_out["ms_per_solve"], 4),
        "unit": "ms/solve",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_out["ms_per_solve"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if args.prec == 0 else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: 3D 7-point variable-coefficient Poisson, Morton order, "
                        f"n={batch.n}, K={batch.K} leaves of 128, {batch.levels} tile levels of rank 32, "
                        f"nnz={batch.nnz}, tol={batch.tol}",
            "vectors": "f64" if args.prec == 0 else "f32", "factors_and_matrix": "f32",
            "scalars": "f64", "x": "f64", "engine": main_out["engine"],
            "iterations": iters, "device": dev_name,
        },
        "iterations_per_s": round(iters / (main_out["ms_per_solve"] * 1e-3), 1),
        "us_per_iteration": round(main_out["ms_per_solve"] * 1e3 / max(iters, 1), 3),
        "apply_us": round(main_out["apply_us"], 3),
        "spmv_us": round(main_out["spmv_us"], 3),
        "apply_spmv_back_to_back_us": round(main_out["pair_back_to_back_us"], 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "M-apply (restrict + prolong) + CSR SpMV, per call",
            "algorithmic_bytes": ab + sb,
        },
        "cpu_baseline": cpu,
        "ms_per_solve_by_config": others,
        "variants_at_workload": variants,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
