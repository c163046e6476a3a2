"""Benchmark: PCG ms/solve and M-apply+SpMV bandwidth against the HBM roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N8k]

A step is one complete H-matrix-preconditioned PCG solve (init, apply, SpMV,
updates and fp64 reductions until ||r|| <= 1e-6 ||b||) of the named workload,
with A, the factors and b already resident in device memory.  The default
workload is the N = 8,192 system (3D 7-point variable-coefficient Poisson on a
16 x 16 x 32 Morton-ordered grid, K = 64 leaves, 6 tile levels).

Printed: one JSON line on stdout.  `value` is ms per solve (lower is better).
`roofline` covers the dominant kernel of the metric's apply + SpMV pair, the
single-pass M-apply: `reps` calls are captured into one graph on the library's
stream and replayed between HIP events on that stream; achieved = algorithmic
bytes (each factor, gate and vector entry read or written once per call) / GPU
time per call, against MI355X's 8 TB/s HBM peak.  Measured warm (the same
factors call after call, served from the Infinity Cache) and cold (factors of
enough copies cycled that they come from HBM), each beside the read ceiling of
one launch over the same bytes from the same place (hpcg_read_probe).  The
pair itself is in `roofline.apply_spmv`.  `cpu_baseline` times the plain C
fp64 oracle on host cores (1 thread and all threads).
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
FP32_MFMA_PEAK_TFLOPS = 157.3
FP16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "PCG ms/solve and M-apply+SpMV HBM GB/s (fraction of peak) at N=8,192"


def apply_bytes(n: int, K: int, levels: int, B: int = 1) -> int:
    """Algorithmic bytes of one M-apply: leaf factors, level slabs, gate, r in, y out."""
    L, R = 128, 32
    return B * 4 * (n * L + n * R * levels + n) + B * 8 * n


def bridge_apply_bytes(n: int, K: int, levels: int, B: int = 1) -> int:
    """Algorithmic bytes of one M-apply in the pages' bridge format: leaf
    factors, the two bridges per leaf, one R x R core per tile, gate, r in, y
    out (the factor part is the packed width of Supplementary Table 3)."""
    L, R = 128, 32
    cores = sum(K >> (l + 1) for l in range(levels))
    return B * 4 * (n * L + (2 * n * R if levels else 0) + cores * R * R + n) + B * 8 * n


def block_apply_flops(n: int, levels: int, nrhs: int, B: int = 1) -> int:
    """Algorithmic flops of one block apply: per column the leaf stage (one
    n x 128 product with the dense leaf blocks F_k = U_k U_k^T), restriction
    and prolongation (two n x 32 products per level) and the gate."""
    L, R = 128, 32
    return B * nrhs * (2 * n * L + 4 * n * R * levels + 2 * n)


def spmv_bytes(n: int, nnz: int, B: int = 1) -> int:
    """Algorithmic bytes of one SpMV: values + column indices, row pointers, x in, y out."""
    return 8 * nnz + 4 * (B * n + 1) + 8 * B * n


# sources of the single-vector apply and SpMV kernels and of their launch code
APPLY_SPMV_SOURCES = ("hpcg_device.hpp", "hpcg_leaf.hpp", "hpcg_apply.hpp")


def kernel_source_digest() -> str:
    """Digest of the apply / SpMV kernel sources, so that recorded counters go
    stale as soon as those kernels or their launch code change."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "matrix_preconditioned_pcg_amd", "csrc")
    for f in APPLY_SPMV_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_record(config: str):
    """HBM bytes per launch of the single-pass apply from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a copy
    kernel's reading), or None when there is none for this workload or the
    kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"apply_traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec.get("apply_bytes_per_launch")


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


def time_calls(fn, reps, stream, torch):
    """Eager timing: mean and median duration of fn() with a HIP event pair
    around every call on `stream` (includes host launch latency)."""
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


def time_graph(fn, reps, stream, torch, replays=5):
    """GPU time per fn() call: `reps` calls captured into one graph on `stream`
    (the library's stream), replayed `replays` times between HIP events on that
    stream; the median replay is reported.  Free of host launch overhead."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(replays):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        e.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(e) * 1e3 / reps)
    del g
    return float(np.median(out))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, budget_s=25.0):
    """The plain C fp64 oracle (oracle/c/pcg_oracle.c) solving the workload on
    host cores: median of up to 21 timed solves after one warm-up, at one
    thread and at every thread OpenMP gets (the box's share of cores); the
    number of solves shrinks so that the whole leg stays near budget_s."""
    from oracle import c_oracle
    sy = batch.system(0)
    args = (sy.row_ptr, sy.col, sy.val, sy.b, sy.U, sy.W, sy.g, batch.tol, batch.maxit)
    all_threads = c_oracle.max_threads()
    per_iter_bytes = apply_bytes(batch.n, batch.K, batch.levels) + spmv_bytes(batch.n, len(sy.col))
    out = {}
    for label, threads in (("one_thread", 1), ("all_threads", all_threads)):
        c_oracle.set_threads(threads)
        t0 = time.perf_counter()
        _x, it, st, _rel = c_oracle.pcg(*args)          # warm-up
        first = time.perf_counter() - t0
        reps = int(max(1, min(21, (budget_s / 2 - first) // max(first, 1e-3))))
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            _x, it, st, _rel = c_oracle.pcg(*args)
            ts.append(time.perf_counter() - t0)
        ms = float(np.median(ts)) * 1e3
        out[label] = {"threads": threads, "ms_per_solve": round(ms, 2), "solves_timed": reps, "iterations": it,
                      "status": st, "iterations_per_s": round(it / ms * 1e3, 1),
                      "apply_spmv_gbs": round(it * per_iter_bytes / ms / 1e6, 2)}
    c_oracle.set_threads(all_threads)
    best = out["all_threads"]
    return {"value": best["ms_per_solve"], "unit": "ms/solve", "cores": best["threads"], "kind": "oracle",
            "sample": f"median of {best['solves_timed']} complete fp64 solves of the {batch.name} system "
                      f"({batch.n} unknowns, {best['iterations']} iterations) by the plain C oracle after one "
                      f"warm-up, at {best['threads']} OpenMP threads; one-thread figure beside it",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "iterations_per_s": best["iterations_per_s"], "one_thread": out["one_thread"],
            "all_threads": out["all_threads"]}


def single_pass_kernel(batch):
    """Which single-pass apply kernel AUTO launches: two workgroups per leaf
    (diagonal / off-diagonal roles) when the batch has at most half as many
    leaves as the device has CUs, else one per leaf."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if 2 * batch.batch * batch.K <= cus:
        return f"M-apply (k_apply_split<{batch.levels}>: one launch, two workgroups per leaf, factors read once)"
    return f"M-apply (k_apply_fused<{batch.levels}>: one launch, one workgroup per leaf, factors read once)"


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
    ap.add_argument("--no-block", action="store_true", help="skip the block (probe) apply timing")
    ap.add_argument("--no-fused", action="store_true", help="skip the forced single-launch apply timing")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the runs with the factors cycled through HBM and the read ceilings (profiling runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run three 256 MiB device-to-device copies (calibrates HBM byte counters)")
    ap.add_argument("--solve-only", action="store_true",
                    help="time only the solves of --config (nothing else runs: a kernel trace of this run "
                         "holds exactly warmup + steps solves)")
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

    # one non-default stream for the library: solves, applies and the graphs
    # that time them all run on it
    stream = torch.cuda.Stream()

    def measure_apply_spmv(batch, solver):
        r = torch.randn(batch.batch * batch.n, device="cuda", dtype=torch.float32)
        y = torch.empty_like(r)
        q = torch.empty_like(r)

        def apply():
            hpcg.hpcg_apply_M(solver.handle, solver.part, r, y)

        def spmv():
            hpcg.hpcg_spmv(solver.handle, solver.part, r, q)

        def pair():
            spmv()
            apply()
        ab = apply_bytes(batch.n, batch.K, batch.levels, batch.batch)
        sb = spmv_bytes(batch.n, batch.nnz, batch.batch)
        fused_us = streaming_us = None
        if not args.no_fused:
            # both apply paths forced, for comparison with what AUTO picks
            solver.set_option(hpcg.HPCG_OPT_APPLY_PATH, hpcg.HPCG_APPLY_STREAMING)
            with torch.cuda.stream(stream):
                streaming_us = time_graph(apply, args.reps, stream, torch)
            if batch.K <= 256:
                solver.set_option(hpcg.HPCG_OPT_APPLY_PATH, hpcg.HPCG_APPLY_FUSED)
                with torch.cuda.stream(stream):
                    fused_us = time_graph(apply, args.reps, stream, torch)
            solver.set_option(hpcg.HPCG_OPT_APPLY_PATH, hpcg.HPCG_APPLY_AUTO)
        with torch.cuda.stream(stream):
            apply()
            torch.cuda.synchronize()
            path = {hpcg.HPCG_APPLY_FUSED: "fused", hpcg.HPCG_APPLY_STREAMING: "streaming"}.get(
                hpcg.hpcg_last_apply_path(solver.handle), "?")
            out = {"apply_us": time_graph(apply, args.reps, stream, torch),
                   "spmv_us": time_graph(spmv, args.reps, stream, torch),
                   "pair_us": time_graph(pair, args.reps, stream, torch)}
            out["apply_us_eager"], _ = time_calls(apply, args.reps, stream, torch)
        out.update(apply_path=path, apply_fused_us=fused_us, apply_streaming_us=streaming_us,
                   apply_bytes=ab, spmv_bytes=sb,
                   apply_gbs=ab / out["apply_us"] / 1e3, spmv_gbs=sb / out["spmv_us"] / 1e3,
                   pair_gbs=(ab + sb) / out["pair_us"] / 1e3)
        out["pair_frac"] = out["pair_gbs"] / HBM_PEAK_GBS
        return out

    def measure_cold(batch, target_bytes=640 << 20):
        """Apply + SpMV pairs, and applies alone, cycling over enough
        independent copies of the system (own workspace, own factor copy) that
        together they exceed the 256 MB Infinity Cache: every call then
        fetches its factors from HBM."""
        ab = apply_bytes(batch.n, batch.K, batch.levels, batch.batch)
        sb = spmv_bytes(batch.n, batch.nnz, batch.batch)
        copies = max(2, int(np.ceil(target_bytes / (ab + sb))))
        dev = [torch.as_tensor(a).cuda() for a in (batch.U, batch.W, batch.g)]
        solvers, vecs = [], []
        for _ in range(copies):
            sv = hpcg.Solver(batch.n, batch.row_ptr, batch.col, batch.val, batch=batch.batch,
                             levels=batch.levels, stream=stream)
            sv.set_factors(*dev)
            solvers.append(sv)
            r = torch.randn(batch.batch * batch.n, device="cuda", dtype=torch.float32)
            vecs.append((r, torch.empty_like(r), torch.empty_like(r)))
        torch.cuda.synchronize()
        state = {"i": 0}

        def pair():
            i = state["i"] % copies
            state["i"] += 1
            r, y, q = vecs[i]
            hpcg.hpcg_spmv(solvers[i].handle, solvers[i].part, r, q)
            hpcg.hpcg_apply_M(solvers[i].handle, solvers[i].part, r, y)

        def apply_only():
            i = state["i"] % copies
            state["i"] += 1
            r, y, _q = vecs[i]
            hpcg.hpcg_apply_M(solvers[i].handle, solvers[i].part, r, y)
        with torch.cuda.stream(stream):
            us = time_graph(pair, 2 * copies, stream, torch)
            us_apply = time_graph(apply_only, 2 * copies, stream, torch)
        for sv in solvers:
            sv.close()
        return {"copies": copies, "bytes_cycled": int(copies * (ab + sb)), "apply_spmv_us": round(us, 3),
                "achieved": round((ab + sb) / us / 1e3, 1), "frac": round((ab + sb) / us / 1e3 / HBM_PEAK_GBS, 4),
                "apply_us": round(us_apply, 3), "apply_gbs": round(ab / us_apply / 1e3, 1),
                "apply_frac": round(ab / us_apply / 1e3 / HBM_PEAK_GBS, 4)}

    def measure_read_ceiling(nbytes, target_bytes=640 << 20):
        """The fastest one-launch read of nbytes (hpcg_read_probe, best of a
        few grid sizes): warm = the same bytes launch after launch (Infinity
        Cache), cold = launches cycling over buffers that together exceed it
        (HBM)."""
        nbytes = (nbytes + 15) // 16 * 16
        copies = max(2, int(np.ceil(target_bytes / nbytes)))
        bufs = [torch.ones(nbytes // 4, device="cuda", dtype=torch.float32) for _ in range(copies)]
        best = {"warm_us": None, "cold_us": None}
        grids = (256, 512, 1024, 2048)
        sinks = {g: torch.empty(g, device="cuda", dtype=torch.float32) for g in grids}
        state = {"i": 0}
        with torch.cuda.stream(stream):
            for g in grids:
                warm = time_graph(lambda: hpcg.hpcg_read_probe(bufs[0], nbytes, sinks[g], g, stream),
                                  args.reps, stream, torch)

                def cyc():
                    i = state["i"] % copies
                    state["i"] += 1
                    hpcg.hpcg_read_probe(bufs[i], nbytes, sinks[g], g, stream)
                cold = time_graph(cyc, 2 * copies, stream, torch)
                if best["warm_us"] is None or warm < best["warm_us"]:
                    best.update(warm_us=warm, warm_grid=g)
                if best["cold_us"] is None or cold < best["cold_us"]:
                    best.update(cold_us=cold, cold_grid=g)
        del bufs
        return {"bytes": nbytes, "warm_us": round(best["warm_us"], 3), "warm_gbs": round(nbytes / best["warm_us"] / 1e3, 1),
                "warm_grid": best["warm_grid"], "cold_us": round(best["cold_us"], 3),
                "cold_gbs": round(nbytes / best["cold_us"] / 1e3, 1), "cold_grid": best["cold_grid"]}

    def measure_launch_floor():
        """Per-call time of the smallest kernel (one workgroup reading 16
        bytes) replayed back to back in a graph: the floor any launch starts
        from."""
        buf = torch.ones(4, device="cuda", dtype=torch.float32)
        sink = torch.empty(1, device="cuda", dtype=torch.float32)
        with torch.cuda.stream(stream):
            return round(time_graph(lambda: hpcg.hpcg_read_probe(buf, 16, sink, 1, stream), args.reps, stream, torch), 3)

    def measure_block(name):
        """Block apply M R on the matrix cores with the pages' probe width
        K_z = max(64, ceil(sqrt(N))) rounded up to 16."""
        batch = make_config(name)
        solver = hpcg.Solver(batch.n, batch.row_ptr, batch.col, batch.val, batch=batch.batch,
                             levels=batch.levels, stream=stream)
        solver.set_factors(batch.U, batch.W, batch.g)
        kz = max(64, int(np.ceil(np.sqrt(batch.n))))
        nrhs = (kz + 15) // 16 * 16
        R = torch.randn(batch.batch * batch.n * nrhs, device="cuda", dtype=torch.float32)
        Y = torch.empty_like(R)
        X = torch.empty_like(R)
        work = torch.empty(hpcg.hpcg_block_workspace_bytes(solver.handle, nrhs), dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(stream):
            t_apply = time_graph(lambda: hpcg.hpcg_apply_M_block(solver.handle, solver.part, R, Y, nrhs, work),
                                 max(20, args.reps // 10), stream, torch)
            t_spmv = time_graph(lambda: hpcg.hpcg_spmv_block(solver.handle, solver.part, R, X, nrhs),
                                max(20, args.reps // 10), stream, torch)
        fl = block_apply_flops(batch.n, batch.levels, nrhs, batch.batch)
        # block PCG on the same block (every column its own solve)
        Bm = torch.randn(batch.batch * batch.n * nrhs, device="cuda", dtype=torch.float32)
        torch.cuda.synchronize()
        solver.solve_block(Bm, nrhs, tol=batch.tol, maxit=batch.maxit)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = 3
        for _ in range(reps):
            _X, its_b, _rel, st_b = solver.solve_block(Bm, nrhs, tol=batch.tol, maxit=batch.maxit)
        torch.cuda.synchronize()
        ms_block = (time.perf_counter() - t0) * 1e3 / reps
        solver.close()
        tf = fl / t_apply / 1e6
        solve = {"ms_per_block_solve": round(ms_block, 3), "status": st_b,
                 "iterations": {"min": min(its_b), "max": max(its_b)},
                 "column_solves_per_s": round(nrhs * batch.batch / ms_block * 1e3, 1)}
        return {"workload": name, "nrhs": nrhs, "probe_columns": kz, "apply_us": round(t_apply, 3),
                "block_solve": solve,
                "tflops": round(tf, 2), "peak_tflops": FP32_MFMA_PEAK_TFLOPS,
                "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4), "flops": fl,
                "dtype": "f32 products from fp16 pairs (mfma 16x16x32 f16, three per f32 product)",
                "f16_mfma_frac": round(3 * tf / FP16_MFMA_PEAK_TFLOPS, 4),
                "spmv_block_us": round(t_spmv, 3)}

    def run_config(name, steps, warmup, with_roofline, engine=None, prec=None):
        batch = make_config(name)
        solver = hpcg.Solver(batch.n, batch.row_ptr, batch.col, batch.val, batch=batch.batch,
                             levels=batch.levels, stream=stream)
        solver.set_factors(batch.U, batch.W, batch.g)
        engine = args.engine if engine is None else engine
        prec = args.prec if prec is None else prec
        if engine:
            solver.set_option(hpcg.HPCG_OPT_ENGINE, engine)
        solver.set_option(hpcg.HPCG_OPT_PRECISION, prec)
        b = torch.as_tensor(batch.b.reshape(-1)).cuda()
        torch.cuda.synchronize()
        ms, iters, res = time_solves(solver, b, batch.tol, batch.maxit, steps, warmup, torch)
        out = {"ms_per_solve": ms, "iterations": iters, "status": res.status,
               "engine": solver.last_engine, "batch": batch.batch, "n": batch.n}
        if with_roofline:
            out.update(measure_apply_spmv(batch, solver))
        solver.close()
        return batch, out

    if args.copy_probe:
        src = torch.ones(64 << 20, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.solve_only:
        batch, o = run_config(args.config, args.steps, args.warmup, False)
        print(json.dumps({"config": args.config, "ms_per_solve": round(o["ms_per_solve"], 4),
                          "solves": args.steps + args.warmup, "iterations": o["iterations"]
                          if len(o["iterations"]) <= 4 else {"min": min(o["iterations"]), "max": max(o["iterations"])},
                          "engine": o["engine"]}))
        return 0
    batch, main_out = run_config(args.config, args.steps, args.warmup, True)
    ab, sb = main_out["apply_bytes"], main_out["spmv_bytes"]
    achieved = main_out["pair_gbs"]
    others = {}
    if not args.no_others:
        for name in CONFIGS:
            if name == args.config:
                continue
            log(f"bench: {name}")
            _b, o = run_config(name, max(3, args.steps // 4), 1, True)
            others[name] = {"ms_per_solve": round(o["ms_per_solve"], 4), "iterations": o["iterations"]
                            if len(o["iterations"]) <= 4 else
                            {"min": min(o["iterations"]), "max": max(o["iterations"])},
                            "engine": o["engine"],
                            "apply_path": o["apply_path"],
                            "apply_us": round(o["apply_us"], 3), "spmv_us": round(o["spmv_us"], 3),
                            "apply_spmv_us": round(o["pair_us"], 3),
                            "apply_spmv_gbs": round(o["pair_gbs"], 1),
                            "apply_spmv_frac": round(o["pair_frac"], 4),
                            "apply_gbs": round(o["apply_gbs"], 1),
                            "apply_frac": round(o["apply_gbs"] / HBM_PEAK_GBS, 4),
                            "spmv_gbs": round(o["spmv_gbs"], 1),
                            "spmv_frac": round(o["spmv_gbs"] / HBM_PEAK_GBS, 4),
                            "residency": "warm (Infinity Cache); peak 8 TB/s HBM"}
            if o["apply_bytes"] + o["spmv_bytes"] >= 8 << 20 and not args.no_cold:
                # also timed with the factors cycled through HBM, and both
                # residencies beside the read ceiling of the apply's bytes
                log(f"bench: {name} cold (factors from HBM) apply + SpMV, read ceilings")
                others[name]["cold"] = measure_cold(_b)
                ceil = measure_read_ceiling(o["apply_bytes"])
                others[name]["read_ceiling"] = ceil
                others[name]["apply_frac_of_warm_ceiling"] = round(o["apply_gbs"] / ceil["warm_gbs"], 4)
                others[name]["apply_frac_of_cold_ceiling"] = round(others[name]["cold"]["apply_gbs"]
                                                                   / ceil["cold_gbs"], 4)
    variants = {}
    if not args.no_variants:
        for label, eng, prec in (("persistent_vec64", 2, 0), ("persistent_vec32", 2, 1),
                                 ("graph_vec64", 1, 0), ("graph_vec32", 1, 1)):
            log(f"bench: variant {label}")
            _b, o = run_config(args.config, max(3, args.steps // 2), 1, False, eng, prec)
            variants[label] = {"ms_per_solve": round(o["ms_per_solve"], 4), "iterations": o["iterations"][0]}
    bridge = None
    if not args.no_variants:
        # the pages' own factor format: bridges + cores, applied natively (and
        # expanded on the device into slabs for the solve)
        from workloads.generate import bridge_factors_for
        bridge = {}
        for name in dict.fromkeys((args.config, "N16k")):
            log(f"bench: bridge-format factors {name}")
            bb = make_config(name)
            Ub, Vb, Bc = bridge_factors_for(bb)
            solver = hpcg.Solver(bb.n, bb.row_ptr, bb.col, bb.val, batch=bb.batch, levels=bb.levels, stream=stream)
            dev = [torch.as_tensor(a).cuda() for a in (bb.U, Ub, Vb, Bc, bb.g)]
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                t_set = time_graph(lambda: hpcg.hpcg_set_factors_bridge(solver.handle, solver.part, *dev), 20,
                                   stream, torch)
            r = torch.randn(bb.batch * bb.n, device="cuda", dtype=torch.float32)
            y = torch.empty_like(r)
            with torch.cuda.stream(stream):
                t_apply = time_graph(lambda: hpcg.hpcg_apply_M(solver.handle, solver.part, r, y), args.reps,
                                     stream, torch)
            path = hpcg.hpcg_last_apply_path(solver.handle)
            bvec = torch.as_tensor(bb.b.reshape(-1)).cuda()
            ms, its, _res = time_solves(solver, bvec, bb.tol, bb.maxit, max(3, args.steps // 2), 1, torch)
            nb = bridge_apply_bytes(bb.n, bb.K, bb.levels, bb.batch)
            bridge[name] = {"set_factors_us": round(t_set, 3), "factor_bytes": int(sum(a.numel() * 4 for a in dev)),
                            "apply_path": "bridge" if path == hpcg.HPCG_APPLY_BRIDGE else str(path),
                            "apply_us": round(t_apply, 3), "apply_bytes": nb,
                            "apply_gbs": round(nb / t_apply / 1e3, 1),
                            "apply_frac": round(nb / t_apply / 1e3 / HBM_PEAK_GBS, 4),
                            "ms_per_solve": round(ms, 4), "iterations": its[0]}
            solver.close()
    tight = None
    if not args.no_variants:
        # rtol 1e-10: fp64 vectors directly, and the outer refinement around
        # fp32-vector inner solves (inner tolerance 1e-5)
        log("bench: tight tolerance")
        bt = make_config(args.config)
        solver = hpcg.Solver(bt.n, bt.row_ptr, bt.col, bt.val, batch=bt.batch, levels=bt.levels, stream=stream)
        solver.set_factors(bt.U, bt.W, bt.g)
        bvec = torch.as_tensor(bt.b.reshape(-1)).cuda()
        ms_d, its_d, _r = time_solves(solver, bvec, 1e-10, 5000, 3, 1, torch)
        solver.set_option(hpcg.HPCG_OPT_PRECISION, hpcg.HPCG_PREC_VEC32)
        solver.solve_refined(bvec, tol=1e-10, maxit=20000, inner_tol=1e-5)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            res_r, outer = solver.solve_refined(bvec, tol=1e-10, maxit=20000, inner_tol=1e-5)
        torch.cuda.synchronize()
        ms_r = (time.perf_counter() - t0) * 1e3 / 3
        tight = {"tol": 1e-10, "vec64_ms_per_solve": round(ms_d, 4), "vec64_iterations": its_d[0],
                 "refined_vec32_ms_per_solve": round(ms_r, 4), "refined_inner_iterations": res_r.iterations[0],
                 "refined_outer_steps": outer[0], "refined_true_relres": res_r.relres[0]}
        solver.close()
    forms = None
    if not args.no_variants:
        # the other preconditioner forms on the workload (graph engine), and
        # factors fitted to A^{-1/2} (squared form) / A^{-1} (direct form)
        from workloads.fitted import fitted_batch
        log("bench: preconditioner forms")
        forms = {}
        bf = make_config(args.config)
        bvec = torch.as_tensor(bf.b.reshape(-1)).cuda()
        for label, form in (("squared", hpcg.HPCG_FORM_SQUARED), ("jacobi", hpcg.HPCG_FORM_JACOBI)):
            solver = hpcg.Solver(bf.n, bf.row_ptr, bf.col, bf.val, batch=bf.batch, levels=bf.levels, stream=stream)
            if form != hpcg.HPCG_FORM_JACOBI:
                solver.set_factors(bf.U, bf.W, bf.g)
            solver.set_option(hpcg.HPCG_OPT_FORM, form)
            ms, its, _r = time_solves(solver, bvec, bf.tol, bf.maxit, max(3, args.steps // 2), 1, torch)
            forms[label] = {"workload": args.config, "ms_per_solve": round(ms, 4), "iterations": its[0],
                            "engine": solver.last_engine}
            solver.close()
        for name in ("N1k", "tet4k"):
            base_b = make_config(name)
            bvec = torch.as_tensor(base_b.b.reshape(-1)).cuda()
            for power, form, label in ((-0.5, hpcg.HPCG_FORM_SQUARED, "fit_inv_sqrt_squared"),
                                       (-1.0, hpcg.HPCG_FORM_DIRECT, "fit_inv_direct")):
                log(f"bench: fitted factors {name} {label}")
                fb = fitted_batch(base_b, power)
                solver = hpcg.Solver(fb.n, fb.row_ptr, fb.col, fb.val, batch=fb.batch, levels=fb.levels,
                                     stream=stream)
                solver.set_factors(fb.U, fb.W, fb.g)
                solver.set_option(hpcg.HPCG_OPT_FORM, form)
                ms, its, _r = time_solves(solver, bvec, fb.tol, fb.maxit, max(3, args.steps // 2), 1, torch)
                lo, hi = solver.estimate_spectrum(60)
                forms[f"{label}_{name}"] = {"ms_per_solve": round(ms, 4), "iterations": its[0],
                                            "engine": solver.last_engine,
                                            "lambda_min_H": round(lo, 6), "lambda_max_H": round(hi, 6)}
                solver.close()
    block = []
    if not args.no_block:
        for name in ("N8k", "N16k"):
            log(f"bench: block apply {name}")
            block.append(measure_block(name))
    if args.no_cold:
        cold = {k: None for k in ("apply_us", "apply_gbs", "apply_frac", "copies", "apply_spmv_us", "achieved",
                                  "frac", "bytes_cycled")}
        ceiling = {"warm_gbs": None, "cold_gbs": None}
        floor_us = None
    else:
        log("bench: cold (factors from HBM) apply + SpMV, read ceilings")
        cold = measure_cold(batch)
        ceiling = measure_read_ceiling(ab)
        floor_us = measure_launch_floor()
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
        "apply_spmv_us": round(main_out["pair_us"], 3),
        "apply_us_eager": round(main_out["apply_us_eager"], 3),
        "apply_fused_us": None if main_out["apply_fused_us"] is None else round(main_out["apply_fused_us"], 3),
        "apply_streaming_us": (None if main_out["apply_streaming_us"] is None
                               else round(main_out["apply_streaming_us"], 3)),
        "roofline": {
            "bound": "hbm",
            "achieved": round(main_out["apply_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(main_out["apply_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic_record(args.config),
            "kernel": (single_pass_kernel(batch) if main_out["apply_path"] == "fused"
                       else "M-apply (k_apply_restrict + k_apply_prolong)")
                      + ", calls graph-replayed back to back on the library stream",
            "bytes_per_launch": ab,
            "us_per_launch": round(main_out["apply_us"], 3),
            "residency": "warm: the same factors call after call, read from the 256 MB Infinity Cache "
                         "(frac is still quoted against the 8 TB/s HBM peak); `cold` has them from HBM",
            "warm_read_ceiling_gbs": ceiling["warm_gbs"],
            "frac_of_warm_read_ceiling": (round(main_out["apply_gbs"] / ceiling["warm_gbs"], 4)
                                          if ceiling["warm_gbs"] else None),
            "launch_floor_us": floor_us,
            "cold": {"apply_us": cold["apply_us"], "achieved": cold["apply_gbs"], "frac": cold["apply_frac"],
                     "cold_read_ceiling_gbs": ceiling["cold_gbs"],
                     "frac_of_cold_read_ceiling": (round(cold["apply_gbs"] / ceiling["cold_gbs"], 4)
                                                   if ceiling["cold_gbs"] else None),
                     "copies_cycled": cold["copies"]},
            "read_ceiling": ceiling,
            "apply_spmv": {
                "kernels": "the apply above + CSR SpMV (k_spmv), pairs graph-replayed back to back",
                "bytes": ab + sb, "us": round(main_out["pair_us"], 3), "achieved": round(achieved, 1),
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "spmv_us": round(main_out["spmv_us"], 3), "spmv_gbs": round(main_out["spmv_gbs"], 1),
                "spmv_frac": round(main_out["spmv_gbs"] / HBM_PEAK_GBS, 4),
                "cold": {k: cold[k] for k in ("apply_spmv_us", "achieved", "frac", "bytes_cycled")}},
            "solve": {
                "kernel": "the whole solve (persistent kernel): iterations x the pair's algorithmic bytes "
                          "per ms of solve, i.e. what an apply + SpMV per iteration would have to stream",
                "effective_gbs": round(iters * (ab + sb) / (main_out["ms_per_solve"] * 1e-3) / 1e9, 1)},
        },
        "cpu_baseline": cpu,
        "by_config": others,
        "variants_at_workload": variants,
        "block_apply": block,
        "bridge_format": bridge,
        "tight_tolerance": tight,
        "preconditioner_forms": forms,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
