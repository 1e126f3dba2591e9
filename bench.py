#!/usr/bin/env python3
"""Benchmark: tree-structured verification of one Gated DeltaNet layer on one MI355X.

A step is one pass of the hot path over one layer's synthetic batch: canopy_tree_verify (tree
preprocessing, S0 projections, masked Gram matrices, triangular solve, read-out) followed by
canopy_commit of a random root-to-leaf path. The serial fork baseline is timed beside it.
Inputs are resident in HBM before the timed region; the timed region holds exactly --steps
steps between two stream synchronisations, timed with HIP events on the launch stream. The
steps are captured once into a HIP graph and the timed region is one replay of it (the kernels
are short enough at B=1 that launching them one by one from Python would time the host);
--eager launches them one by one instead.

Prints one JSON line. The default workload is the 9B-shaped layer: B=1, H=32, d=128, T=16
top-k tree (root, 3 children, 4 children each), bf16 q/k/v, fp32 state.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per GDN layer tree-verify (+nodes/s) at B=1/16, T=16-256; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA

WORKLOADS = {
    "binary7_fp32": dict(B=1, H=2, T=7, tree="binary7", dtype="fp32", seed=0,
                         desc="B=1 H=2 T=7 balanced binary tree, fp32 q/k/v"),
    "topk16_b1": dict(B=1, H=32, T=16, tree="topk", tree_kw={"branching": (3, 4)}, dtype="bf16",
                      seed=1, desc="B=1 H=32 T=16 top-k tree 1+3+12, bf16 q/k/v, fp32 S0"),
    "skewed64_b16": dict(B=16, H=32, T=64, tree="skewed", dtype="bf16", seed=2,
                         desc="B=16 H=32 T=64 skewed trees, bf16 q/k/v, fp32 S0"),
    "random256_b16": dict(B=16, H=32, T=256, tree="random", dtype="bf16", seed=3,
                          desc="B=16 H=32 T=256 random recursive trees, bf16 q/k/v, fp32 S0"),
}
for _B in (1, 2, 4, 8):
    WORKLOADS[f"skewed64_b{_B}"] = dict(B=_B, H=32, T=64, tree="skewed", dtype="bf16", seed=2,
                                        desc=f"B={_B} H=32 T=64 skewed trees, bf16 q/k/v, fp32 S0")


def verify_bytes(B, H, T, dtype):
    """Algorithmic HBM bytes of one verify launch: S0 once per (sequence, head), then per node
    and head q, k, v (input dtype), alpha and beta (fp32), O and U (fp32) and ell (fp32), plus
    the parent array."""
    ib = 2 if dtype == "bf16" else 4
    per_node_head = 3 * 128 * ib + 8 + 2 * 128 * 4 + 4
    return B * H * (128 * 128 * 4 + T * per_node_head) + B * T * 4


def commit_bytes(B, H, m_total):
    """S0 read and S_new written per (sequence, head), plus k (bf16) and U rows and alpha of
    the path nodes (m_total path nodes summed over sequences), plus the path arrays."""
    return B * H * 2 * 128 * 128 * 4 + m_total * H * (128 * 2 + 128 * 4 + 4) + m_total * 8


def build_inputs(wl):
    import synth
    kw = {k: wl[k] for k in ("B", "H", "T", "tree", "dtype", "seed")}
    return synth.make_inputs(tree_kw=wl.get("tree_kw"), **kw)


def to_device(inp):
    import numpy as np
    import torch
    out = {}
    if inp["dtype"] == "bf16":
        for n in ("q", "k", "v"):
            out[n] = torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
    else:
        for n in ("q", "k", "v"):
            out[n] = torch.from_numpy(inp[n]).cuda()
    for n in ("alpha", "beta", "S0"):
        out[n] = torch.from_numpy(inp[n]).cuda()
    for n in ("parent", "path", "path_len"):
        out[n] = torch.from_numpy(inp[n].astype(np.int32)).cuda()
    return out


def graph_of(fn, n):
    """A HIP graph holding n back-to-back calls of fn (captured on torch's capture stream, which
    is the stream the library launches on)."""
    import torch
    fn()  # warm the caching allocator and the code objects outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, n):
    """Average µs per call of a graph of n calls: one replay between two events on the stream
    the replay runs on, synchronised on both sides."""
    import torch
    g.replay()  # warm replay
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / n


def time_eager(fn, iters, warmup):
    """Average µs per call of fn() over `iters` back-to-back eager calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / iters


def cpu_baseline(inp, budget_s=10.0):
    """The oracle (fp64 per-path recurrence + path commit) timed on the host cores on the same
    workload, repeated until about `budget_s` seconds: µs per layer."""
    import oracle
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.gdn_tree(inp["parent"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                        inp["S0"])
        oracle.commit(inp["parent"], inp["path"], inp["path_len"], inp["k"], inp["v"],
                      inp["alpha"], inp["beta"], inp["S0"])
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s and len(times) >= 3:
            break
        if len(times) >= 1 and times[0] > budget_s:
            break
    times.sort()
    med = times[len(times) // 2]
    return dict(value=med * 1e6, unit="us per layer (verify + commit)", cores=oracle.num_threads(),
                kind="oracle", sample=f"{len(times)} full layers of this workload, median")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default="topk16_b1", choices=sorted(WORKLOADS))
    ap.add_argument("--solver", default="auto", choices=["auto", "fwdsub", "neumann", "level"])
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-serial", action="store_true", help="skip the serial fork baseline")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying a HIP graph")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify and commit kernels shard by (sequence, "
              "head) with no exchange, and this build runs on a single MI355X. Use --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import tree_speculative_verification_amd as tsv

    wl = WORKLOADS[args.workload]
    B, H, T, dt = wl["B"], wl["H"], wl["T"], wl["dtype"]
    inp = build_inputs(wl)
    d = to_device(inp)
    tsv.load()
    O = torch.empty((B, T, H, 128), device="cuda")
    U = torch.empty_like(O)
    ell = torch.empty((B, T, H), device="cuda")
    S_new = torch.empty_like(d["S0"])

    def verify():
        tsv.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                        solver=args.solver, waves=args.waves, out=(O, U, ell))

    def commit():
        tsv.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"], out=S_new)

    def step():
        verify()
        commit()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref_O, ref_U, ref_S = O.clone(), U.clone(), S_new.clone()
    if args.eager:
        us_step = time_eager(step, args.steps, 0)
        us_verify = time_eager(verify, args.steps, 5)
        us_commit = time_eager(commit, args.steps, 5)
    else:
        # Timed region: one replay of a graph holding exactly `steps` steps.
        g_step = graph_of(step, args.steps)
        us_step = time_graph(g_step, args.steps)
        # The replayed kernels must reproduce the eager results bit for bit.
        if not (torch.equal(O, ref_O) and torch.equal(U, ref_U) and torch.equal(S_new, ref_S)):
            raise RuntimeError("graph replay differs from the eager run")
        del g_step
        g_v = graph_of(verify, args.steps)
        us_verify = time_graph(g_v, args.steps)
        del g_v
        g_c = graph_of(commit, args.steps)
        us_commit = time_graph(g_c, args.steps)
        del g_c
    us_serial = None
    if not args.no_serial:
        snaps = torch.empty((B, T, H, 128, 128), device="cuda")

        def serial():
            tsv.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                              snapshots=snaps)
        n_ser = max(10, args.steps // 4)
        if args.eager:
            us_serial = time_eager(serial, n_ser, 3)
        else:
            g_s = graph_of(serial, n_ser)
            us_serial = time_graph(g_s, n_ser)
            del g_s
        del snaps

    vbytes = verify_bytes(B, H, T, dt)
    achieved = vbytes / (us_verify * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(us_step, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "B": B, "H": H, "T": T, "dk": 128, "dv": 128,
                   "tree": wl["tree"], "solver": args.solver, "waves": args.waves,
                   "step": "verify + commit of a random root-to-leaf path",
                   "launch": "eager" if args.eager else "hip graph of all timed steps"},
        "nodes_per_s": round(B * T / (us_step * 1e-6), 1),
        "verify_us": round(us_verify, 3),
        "verify_nodes_per_s": round(B * T / (us_verify * 1e-6), 1),
        "commit_us": round(us_commit, 3),
        "serial_verify_us": None if us_serial is None else round(us_serial, 3),
        "roofline": {"bound": "hbm", "kernel": "verify_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": None, "algorithmic_bytes": vbytes},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
