"""In-kernel timeline of the single-pass apply and the SpMV (a measurement aid).

    python -m matrix_preconditioned_pcg_amd.timeline [--config N16k] [--build] [--calls 200]
    python -m matrix_preconditioned_pcg_amd.timeline --config N8k --block 96

Runs the HPCG_TRACE build of the library (libhpcg_trace.so, compiled first
with --build or when missing): the kernels record thread 0's reading of the
constant 100 MHz real-time counter at fixed points of their work.  `--calls`
applies (or SpMVs) are captured into one graph and replayed, so the stamps read
afterwards are those of a call that ran right behind another, as in a
benchmark.  For every stamp the script prints the distribution over
workgroups of the time since the earliest workgroup start of that call, in
microseconds, as a markdown table.
"""

from __future__ import annotations

import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SLOTS = 16
TICK_US = 0.01          # 100 MHz

FUSED = {0: "start", 1: "r in LDS (first load back)", 2: "restriction published",
         3: "U_k^T r reduced", 4: "diagonal stage done", 10: "first poll of the partner words back",
         5: "partner words gathered", 8: "strip sums done", 9: "off-diagonal prolongation done",
         6: "prolongation done", 7: "y stored and acknowledged"}
SPLIT_DIAG = {0: "start", 1: "r in LDS", 2: "U_k U_k^T r published"}
SPLIT_OFF = {0: "start", 1: "r in LDS", 2: "restriction published",
             5: "partner + diagonal words gathered", 6: "prolongation done", 7: "y stored and acknowledged"}
SPMV = {0: "start", 7: "y stored and acknowledged"}
BLOCK_LEAF = {0: "start", 1: "R tile and operands landed", 2: "R^T in LDS (and the block solve's update)",
              6: "Y = F_k R + g R stores issued"}
BLOCK_RESTR = {0: "start", 1: "R tile and operands landed", 2: "the block solve's update done",
               4: "restrictions stored"}
BLOCK_BOTH = {0: "start", 1: "R tile and operands landed", 2: "R^T in LDS (and the block solve's update)",
              6: "Y = F_k R + g R stores issued", 4: "restrictions stored"}
BLOCK_PROLONG = {8: "start", 9: "half sums in LDS", 10: "products done", 11: "Y stores issued"}
RESIDENT = {0: "iteration start", 1: "halo z and r.r, r.z partials polled", 2: "SpMV done",
            3: "restriction of q and p.q published", 4: "U_k U_k^T q done",
            5: "partners' W^T q and p.q polled", 6: "alpha, r, x and z = M r done", 7: "exact refresh (when due)",
            8: "z and partials published"}


def table(title, stamps, names, t0):
    rows = [f"**{title}** ({stamps.shape[0]} workgroups; us since the earliest start)", "",
            "| stamp | min | median | max |", "|---|---|---|---|"]
    for slot, name in names.items():
        if not stamps[:, slot].any():
            continue   # a point this kernel does not stamp (the bridge apply has no separate off-diagonal one)
        v = (stamps[:, slot].astype(np.int64) - t0) * TICK_US
        rows.append(f"| {name} | {v.min():.2f} | {np.median(v):.2f} | {v.max():.2f} |")
    return "\n".join(rows)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="N16k")
    ap.add_argument("--calls", type=int, default=200)
    ap.add_argument("--build", action="store_true")
    ap.add_argument("--bridge", action="store_true", help="factors in the bridge format (native bridge apply)")
    ap.add_argument("--solve", action="store_true", help="also one resident solve: its 66th iteration")
    ap.add_argument("--block", type=int, default=0, metavar="NRHS",
                    help="instead: the block apply's leaf stage and prolongation on NRHS columns, in a "
                         "replayed graph of block applies and in the last iteration of a block solve")
    args = ap.parse_args(argv)
    from matrix_preconditioned_pcg_amd import build as build_mod
    if args.build or not os.path.exists(build_mod.TRACE_LIB):
        build_mod.build(trace=True)
    os.environ["HPCG_LIBRARY"] = build_mod.TRACE_LIB

    import torch

    from matrix_preconditioned_pcg_amd import hpcg
    from workloads import make_config

    assert torch.cuda.is_available(), "the timeline needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    batch = make_config(args.config)
    solver = hpcg.Solver(batch.n, batch.row_ptr, batch.col, batch.val, batch=batch.batch, levels=batch.levels,
                         stream=stream)
    if args.bridge:
        from workloads.generate import bridge_factors_for
        solver.set_factors_bridge(batch.U, *bridge_factors_for(batch), batch.g)
    else:
        solver.set_factors(batch.U, batch.W, batch.g)
    r = torch.randn(batch.batch * batch.n, device="cuda", dtype=torch.float32)
    y = torch.empty_like(r)
    q = torch.empty_like(r)

    def replay(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(args.calls):
                fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        hpcg.hpcg_trace_read(0, clear=True)
        g.replay()
        torch.cuda.synchronize()
        del g

    if args.block:
        solver.close()
        return block_timeline(args, batch, stream, hpcg, torch)
    fmt = " --bridge" if args.bridge else ""
    out = [f"# In-kernel timeline, {args.config} (n = {batch.n}, K = {batch.K}, {batch.levels} levels, "
           f"batch {batch.batch}){', bridge-format factors' if args.bridge else ''}", "",
           f"Command: `python -m matrix_preconditioned_pcg_amd.timeline --config {args.config}{fmt} --build`", ""]
    with torch.cuda.stream(stream):
        replay(lambda: hpcg.hpcg_apply_M(solver.handle, solver.part, r, y))
    path = hpcg.hpcg_last_apply_path(solver.handle)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    items = batch.batch * batch.K
    st = np.array(hpcg.hpcg_trace_read(4096 * SLOTS), dtype=np.uint64).reshape(4096, SLOTS)
    single = path in (hpcg.HPCG_APPLY_FUSED, hpcg.HPCG_APPLY_BRIDGE)
    if single and 2 * items <= ncu:
        wg = st[:2 * items]
        t0 = int(wg[:, 0].astype(np.int64).min())
        out.append(table("single-pass apply, two workgroups per leaf: diagonal role", wg[0::2], SPLIT_DIAG, t0))
        out += ["", table("single-pass apply, two workgroups per leaf: off-diagonal role", wg[1::2], SPLIT_OFF, t0)]
        span = (int(wg[1::2, 7].astype(np.int64).max()) - t0) * TICK_US
    elif single:
        wg = st[:min(items, ncu)]
        t0 = int(wg[:, 0].astype(np.int64).min())
        out.append(table("single-pass apply, one workgroup per leaf", wg, FUSED, t0))
        span = (int(wg[:, 7].astype(np.int64).max()) - t0) * TICK_US
    else:
        print("the apply did not take the single-pass path", file=sys.stderr)
        return 1
    out += ["", f"Apply: first workgroup start to last acknowledged store {span:.2f} us.", ""]
    with torch.cuda.stream(stream):
        replay(lambda: hpcg.hpcg_spmv(solver.handle, solver.part, r, q))
    nwg = (batch.batch * batch.n + 63) // 64
    sp = np.array(hpcg.hpcg_trace_read(min(nwg, 4096) * SLOTS), dtype=np.uint64).reshape(-1, SLOTS)
    t0 = int(sp[:, 0].astype(np.int64).min())
    out.append(table("CSR SpMV (k_spmv)", sp, SPMV, t0))
    out += ["", f"SpMV: first workgroup start to last acknowledged store "
                f"{(int(sp[:, 7].astype(np.int64).max()) - t0) * TICK_US:.2f} us."]
    if args.solve:
        b = torch.as_tensor(batch.b.reshape(-1)).cuda()
        with torch.cuda.stream(stream):
            solver.solve(b)
            torch.cuda.synchronize()
            hpcg.hpcg_trace_read(0, clear=True)
            res = solver.solve(b)
            torch.cuda.synchronize()
        if hpcg.hpcg_last_engine(solver.handle) == hpcg.HPCG_ENGINE_PERSISTENT and min(res.iterations) > 66:
            nwg = min(items, ncu)
            rs = np.array(hpcg.hpcg_trace_read(nwg * SLOTS), dtype=np.uint64).reshape(nwg, SLOTS)
            t0 = int(rs[:, 0].astype(np.int64).min())
            out += ["", table(f"resident solve, iteration 66 of {res.iterations[0]} (first launch)", rs,
                              RESIDENT, t0)]
            d = np.diff(rs[:, [0, 1, 2, 3, 4, 5, 6, 7, 8]].astype(np.int64), axis=1) * TICK_US
            names = list(RESIDENT.values())
            out += ["", "Per workgroup, median time between consecutive stamps (us):", "",
                    "| from | to | median |", "|---|---|---|"]
            out += [f"| {names[i]} | {names[i + 1]} | {np.median(d[:, i]):.2f} |" for i in range(d.shape[1])]
    solver.close()
    print("\n".join(out))
    return 0


def block_tables(st, items, title):
    """Tables of the leaf-stage kernel (by role) and of the prolongation."""
    role = st[:, 7].astype(np.int64)
    split = bool(np.any(role[:2 * items] == 1))
    nwg = 2 * items if split else items
    wg = st[:nwg]
    t0 = int(wg[:, 0].astype(np.int64).min())
    out = []
    if split:
        r = role[:nwg]
        out += [table(f"{title}: leaf stage (role 0 of two workgroups per item)", wg[r == 0], BLOCK_LEAF, t0), "",
                table(f"{title}: restriction (role 1)", wg[r == 1], BLOCK_RESTR, t0), ""]
        end = max(int(wg[r == 0][:, 6].astype(np.int64).max()), int(wg[r == 1][:, 4].astype(np.int64).max()))
    else:
        out += [table(f"{title}: leaf stage and restriction (one workgroup per item)", wg, BLOCK_BOTH, t0), ""]
        end = int(wg[:, [4, 6]].astype(np.int64).max())
    out += [f"Leaf-stage kernel: first start to its last store issued {(end - t0) * TICK_US:.2f} us.", ""]
    pw = st[:items]
    t1 = int(pw[:, 8].astype(np.int64).min())
    out += [table(f"{title}: prolongation", pw, BLOCK_PROLONG, t1), "",
            f"Prolongation: first start to last Y store issued "
            f"{(int(pw[:, 11].astype(np.int64).max()) - t1) * TICK_US:.2f} us.", ""]
    return out


def block_timeline(args, batch, stream, hpcg, torch):
    nrhs = args.block
    solver = hpcg.Solver(batch.n, batch.row_ptr, batch.col, batch.val, batch=batch.batch, levels=batch.levels,
                         stream=stream)
    solver.set_factors(batch.U, batch.W, batch.g)
    R = torch.randn(batch.batch * batch.n * nrhs, device="cuda", dtype=torch.float32)
    Y = torch.empty_like(R)
    work = torch.empty(hpcg.hpcg_block_workspace_bytes(solver.handle, nrhs), dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        fn = lambda: hpcg.hpcg_apply_M_block(solver.handle, solver.part, R, Y, nrhs, work)  # noqa: E731
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(max(1, args.calls // 10)):
                fn()
        g.replay()
        torch.cuda.synchronize()
        hpcg.hpcg_trace_read(0, clear=True)
        g.replay()
        torch.cuda.synchronize()
        del g
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    # items = (system, leaf, column tile) workgroups of the kernels: read enough rows
    st = np.array(hpcg.hpcg_trace_read(4096 * SLOTS), dtype=np.uint64).reshape(4096, SLOTS)
    items = int(np.count_nonzero(st[:, 8]))
    out = [f"# In-kernel timeline of the block apply, {args.config} (n = {batch.n}, K = {batch.K}, "
           f"{batch.levels} levels, batch {batch.batch}), {nrhs} columns", "",
           f"Command: `python -m matrix_preconditioned_pcg_amd.timeline --config {args.config} --block {nrhs} "
           f"--build`", "", f"{items} (leaf, column tile) items on {ncu} compute units.", ""]
    out += block_tables(st, items, "block apply")
    Bm = torch.randn(batch.batch * batch.n * nrhs, device="cuda", dtype=torch.float32)
    solver.solve_block(Bm, nrhs, tol=batch.tol, maxit=batch.maxit)
    torch.cuda.synchronize()
    hpcg.hpcg_trace_read(0, clear=True)
    _x, its, _rel, _st = solver.solve_block(Bm, nrhs, tol=batch.tol, maxit=batch.maxit)
    torch.cuda.synchronize()
    st = np.array(hpcg.hpcg_trace_read(4096 * SLOTS), dtype=np.uint64).reshape(4096, SLOTS)
    out += [f"Block solve ({min(its)}-{max(its)} iterations): the last iteration's kernels.", ""]
    out += block_tables(st, items, "block solve")
    solver.close()
    print("\n".join(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
