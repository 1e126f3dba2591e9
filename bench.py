#!/usr/bin/env python3
"""Benchmark: tree-structured verification of one Gated DeltaNet layer on one MI355X.

A step is one pass of the hot path over one layer's synthetic batch, as a decode loop runs it:
canopy_commit_verify commits the previous round's accepted path (a random root-to-leaf path of
the tree) into the state the loop carries, then verifies the tree from the committed state
(tree preprocessing, S0 projections, masked Gram matrices, triangular solve, read-out). For
trees of at most 16 nodes, and of 17 to 64 at small batch, that is one launch; otherwise the
commit kernel and the verify kernel.
The same work as two separate calls (canopy_tree_verify, then canopy_commit) is timed beside
it, and so is the serial fork baseline. Inputs are resident in HBM before the timed region; the
timed region holds exactly --steps steps between two stream synchronisations, timed with HIP
events on the launch stream. The steps are captured once into a HIP graph and the timed region
is one replay of it (the kernels are short enough at B=1 that launching them one by one from
Python would time the host), after untimed replays of at least 30 ms of GPU time that let the
clocks settle; --eager launches them one by one instead.

Prints one JSON line. The default workload is the 9B-shaped layer: B=1, H=32, d=128, T=16
top-k tree (root, 3 children, 4 children each), bf16 q/k/v, fp32 state.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per GDN layer tree-verify (+nodes/s) at B=1/16, T=16-256; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
# HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE), keyed by the
# digest of the kernel sources they were taken on; ignored once the sources have changed.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCE_DIR = os.path.join(ROOT, "tree_speculative_verification_amd", "csrc")

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
WORKLOADS["topk16_b16"] = dict(B=16, H=32, T=16, tree="topk", tree_kw={"branching": (3, 4)}, dtype="bf16",
                              seed=1, desc="B=16 H=32 T=16 top-k trees 1+3+12, bf16 q/k/v, fp32 S0")
DEFAULT_WORKLOAD = "topk16_b1"
# Timed beside the default workload in every default run.
EXTRA_WORKLOADS = ("random256_b16", "topk16_b16")
# Grouped value heads ("Qwen3.5-9B shapes": 16 q/k heads serving 32 value heads) and a ragged
# batch (each sequence's own node count, drawn uniformly from the given range).
WORKLOADS["topk16_b1_hk16"] = dict(B=1, H=32, HK=16, T=16, tree="topk", tree_kw={"branching": (3, 4)},
                                   dtype="bf16", seed=1,
                                   desc="B=1 H=32 value heads, 16 q/k heads, T=16 top-k tree 1+3+12, bf16 q/k/v, fp32 S0")
WORKLOADS["random256_b16_hk16"] = dict(B=16, H=32, HK=16, T=256, tree="random", dtype="bf16", seed=3,
                                       desc="B=16 H=32 value heads, 16 q/k heads, T=256 random recursive trees, bf16 q/k/v, fp32 S0")
WORKLOADS["random256_b16_ragged"] = dict(B=16, H=32, HK=16, T=256, tree="random", dtype="bf16", seed=5,
                                         ragged=(64, 256),
                                         desc="B=16 H=32 value heads, 16 q/k heads, ragged random trees of 64-256 nodes (T=256), bf16 q/k/v, fp32 S0")
for _B in (1, 2, 4, 8):
    WORKLOADS[f"skewed64_b{_B}"] = dict(B=_B, H=32, T=64, tree="skewed", dtype="bf16", seed=2,
                                        desc=f"B={_B} H=32 T=64 skewed trees, bf16 q/k/v, fp32 S0")
    WORKLOADS[f"random256_b{_B}"] = dict(B=_B, H=32, T=256, tree="random", dtype="bf16", seed=3,
                                         desc=f"B={_B} H=32 T=256 random recursive trees, bf16 q/k/v, fp32 S0")
    WORKLOADS[f"random128_b{_B}"] = dict(B=_B, H=32, T=128, tree="random", dtype="bf16", seed=4,
                                         desc=f"B={_B} H=32 T=128 random recursive trees, bf16 q/k/v, fp32 S0")


def verify_bytes(B, H, T, dtype, HK=None, nodes=None):
    """Algorithmic HBM bytes of one verify launch: S0 once per (sequence, value head), then per
    node and value head v (input dtype), alpha and beta (fp32), O and U (fp32) and ell (fp32),
    per node and q/k head q and k (input dtype; HK = H when every value head has its own), plus
    the parent array. ``nodes`` is the batch's real node count (B * T unless ragged)."""
    ib = 2 if dtype == "bf16" else 4
    HK = H if HK is None else HK
    nodes = B * T if nodes is None else nodes
    per_node = H * (128 * ib + 8 + 2 * 128 * 4 + 4) + HK * 2 * 128 * ib
    return B * H * 128 * 128 * 4 + nodes * per_node + B * T * 4


def commit_bytes(B, H, m_total):
    """S0 read and S_new written per (sequence, head), plus k (bf16) and U rows and alpha of
    the path nodes (m_total path nodes summed over sequences), plus the path arrays."""
    return B * H * 2 * 128 * 128 * 4 + m_total * H * (128 * 2 + 128 * 4 + 4) + m_total * 8


def fused_step_bytes(B, H, T, dtype, m_total, HK=None, nodes=None):
    """Algorithmic HBM bytes of the one-launch decode step: the verify's bytes plus the commit's,
    with S0 read once for both (the committed state goes from registers into the verify)."""
    return verify_bytes(B, H, T, dtype, HK=HK, nodes=nodes) + commit_bytes(B, H, m_total) - B * H * 128 * 128 * 4


def _mid_col_tiles(heads, waves):
    """The 17-64-node kernel's 16-column tiles per workgroup, as the library picks them."""
    if waves:
        return 4 if waves == 8 else waves
    return 1 if heads <= 32 else (2 if heads <= 64 else 4)


def _step_col_tiles(T, heads, waves):
    """The column tiles canopy_commit_verify gives the 17-64-node kernel: as the verify alone,
    except 2 (the one-launch form) at 49-64 nodes and 65-128 heads with waves 0."""
    if waves == 0 and T > 48 and 64 < heads <= 128:
        return 2
    return _mid_col_tiles(heads, waves)


def one_launch_step(T, solver, heads=32, waves=0):
    """Whether canopy_commit_verify runs the step as one launch (after previous trees of at most
    64 nodes): trees of at most 16 nodes (AUTO, NEUMANN), and trees of 17 to 64 nodes (not
    LEVEL) whose workgroups hold at most 2 state pairs per thread (4 * tiles <= 2 * sub-blocks)."""
    if solver in ("series", "squaring", "split", "levelsync"):
        return False
    if T <= 16:
        return solver in ("auto", "neumann")
    if T <= 64 and solver != "level":
        return 4 * _step_col_tiles(T, heads, waves) <= 2 * ((T + 15) // 16)
    return False


def small_width(heads, waves, fuse, dtype="bf16"):
    """(waves per workgroup, column tiles per wave) of the T <= 16 kernel, as the library picks
    them: waves 16 is single-wave workgroups on two column tiles; waves 0 takes two tiles for
    bf16 inputs once single-tile waves fill one pass or more (3 per SIMD for the one-launch
    step, 4 for the verify alone, on 1024 SIMDs)."""
    if waves == 0:
        waves = 16 if dtype == "bf16" and heads * 8 >= 1024 * (3 if fuse else 4) else 1
    return (1, 2) if waves == 16 else (waves, 1)


def fused_kernel_name(T, dtype="bf16", heads=32, waves=0):
    """The one-launch step's kernel as the profiler names it."""
    bf = "true" if dtype == "bf16" else "false"
    if T <= 16:
        nwv, nct = small_width(heads, waves, True, dtype)
        return "canopy::verify_small_kernel<%s, %d, true, %d>" % (bf, nwv, nct)
    return "canopy::verify_mid_kernel<%s, %d, %d, true>" % (bf, (T + 15) // 16, _step_col_tiles(T, heads, waves))


def verify_flops_ragged(H, lens):
    """verify_flops summed over sequences of their own node counts."""
    return sum(verify_flops(1, H, int(n)) for n in lens)


def verify_flops(B, H, T):
    """Dense-triangle matrix flops of one verify launch: the Gram, solve and read-out matrices
    counted as whole lower triangles, as a tiled kernel issues them (a tree's ancestor pattern
    is sparser, so this is not the method's count): per (sequence, head) the projections K S0
    and Q S0 (4 T d^2), the strict and inclusive Gram triangles (2 d T^2 together), the
    triangular solve and the C U read-out (2 d T^2 together)."""
    d = 128
    return B * H * (4 * T * d * d + 4 * d * T * T)


def ancestor_pairs(parent, n=None):
    """|A| = sum over the first n nodes of |A(i)|, the number of (node, strict ancestor) pairs
    (depth by the parent walk, parents before children)."""
    n = len(parent) if n is None else int(n)
    depth = [0] * n
    for i in range(n):
        p = int(parent[i])
        depth[i] = depth[p] + 1 if p >= 0 else 0
    return sum(depth)


def method_flops(parents, H, lens=None):
    """The method's own matrix flops for one verify launch, from each tree's ancestor pairs:
    per (sequence, head) the projections K S0 and Q S0 (4 T d^2), G over strict ancestors
    (2 |A| d), C over paths (2 (|A| + T) d), the substitution over strict ancestors (2 |A| d)
    and the read-out over paths (2 (|A| + T) d)."""
    d = 128
    tot = 0
    for b, par in enumerate(parents):
        n = len(par) if lens is None else int(lens[b])
        A = ancestor_pairs(par, n)
        tot += 4 * n * d * d + 8 * A * d + 4 * n * d
    return H * tot


def commit_flops(H, m_total):
    """Flops of the commit's rank-m update: 2 d^2 per path node and head."""
    return H * 2 * 128 * 128 * m_total


def verify_kernel_name(T, solver, heads=0, waves=0, dtype="bf16"):
    """The kernel canopy_tree_verify launches for this size, solver, head count and width."""
    if solver in ("series", "squaring", "split"):
        return "mat_apply_kernel"
    if solver == "levelsync":
        return "verify_kernel"
    if T <= 16 and solver in ("auto", "neumann"):
        return "verify_small_kernel"
    if 16 < T <= 64 and solver != "level":
        return "verify_mid_kernel"
    if T > 64 and dtype == "bf16" and solver in ("auto", "fwdsub"):
        if waves in (1, 2) or (waves == 0 and heads <= 128):
            return "verify_wide_kernel"
        if waves == 16 or (waves == 0 and heads > 256):
            return "verify_dual_kernel"
    return "verify_kernel"


def _code_only(text):
    """C++ source with comments removed and whitespace runs collapsed (string literals, which the
    kernels do not use, are not special-cased)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_digest():
    """Digest of the device code (every HIP source and header but the host-side C ABI file, with
    comments and whitespace left out): identifies the kernels a profile was taken on."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(KERNEL_SOURCE_DIR)):
        if f.endswith((".hip", ".hpp")) and f != "api.hip":
            h.update(f.encode())
            with open(os.path.join(KERNEL_SOURCE_DIR, f), encoding="utf-8") as fh:
                h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, solver, waves, role="verify"):
    """HBM bytes per launch of the verify, commit or one-launch step ("fused") kernel from the
    committed counter summary, or None if there is none for this configuration or the kernels
    have changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("kernel_digest") != kernel_digest():
        return None
    ent = data.get("workloads", {}).get(f"{workload}:{solver}:{waves}")
    if ent is None or role not in ent:
        return None
    return ent[role]["hbm_bytes_per_launch"]


def pmc_summary(run_dir, out_path):
    """Turn rocprofv3 --pmc runs of bench.py (one per counter and workload, each with
    --copy-probe) into the per-launch HBM traffic summary. FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) are scaled by what the same counter reads for the probe's plain copy of known
    size."""
    def per_kernel(path):
        acc = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    out = {"kernel_digest": None, "workloads": {}, "note": (
        "HBM bytes per launch = FETCH_SIZE KiB x 1024 x fetch_scale + WRITE_SIZE KiB x 1024 x "
        "write_scale, each scale = probe copy bytes / what the counter reads for that copy")}
    for name in sorted(os.listdir(run_dir)):
        if not name.startswith("pmc_FETCH_SIZE_") or not os.path.isdir(os.path.join(run_dir, name)):
            continue
        tag = name[len("pmc_FETCH_SIZE_"):]
        fdir, wdir = os.path.join(run_dir, name), os.path.join(run_dir, "pmc_WRITE_SIZE_" + tag)
        with open(fdir + ".log") as fh:
            line = next(l for l in fh if l.startswith("{"))
        rec = json.loads(line)
        probe = rec["config"]["copy_probe_bytes"]
        if out["kernel_digest"] is None:
            out["kernel_digest"] = rec["kernel_digest"]
        elif out["kernel_digest"] != rec["kernel_digest"]:
            raise RuntimeError(f"{tag}: counters taken on different kernel sources")
        f = per_kernel(os.path.join(fdir, "run_counter_collection.csv"))
        w = per_kernel(os.path.join(wdir, "run_counter_collection.csv"))
        fscale = probe / 1024.0 / max(f["__amd_rocclr_copyBuffer"])
        wscale = probe / 1024.0 / max(w["__amd_rocclr_copyBuffer"])
        ent = {"config": rec["config"], "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)}
        def is_fused(k):
            # the FUSE argument: third of verify_small_kernel<BF, NWV, FUSE, NCT>, last of
            # verify_mid_kernel<BF, NSB, NCT, FUSE>
            return re.match(r"void canopy::(verify_small_kernel<\w+, \d+, true[,>]|"
                            r"verify_mid_kernel<\w+, \d+, \d+, true>)", k) is not None
        roles = (("verify", lambda k: k.startswith("void canopy::verify") and not is_fused(k), True),
                 ("commit", lambda k: k.startswith("void canopy::commit_kernel<"), True),
                 ("fused", is_fused, False))
        for role, match, required in roles:
            kf = [k for k in f if match(k)]
            if not kf and not required:
                continue
            if len(kf) != 1:
                raise RuntimeError(f"{tag}: expected one {role} kernel in the counters, found {kf}")
            fk = sum(f[kf[0]]) / len(f[kf[0]])
            wk = sum(w[kf[0]]) / len(w[kf[0]])
            ent[role] = {"kernel": kf[0], "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                         "hbm_bytes_per_launch": int(round(fk * 1024 * fscale + wk * 1024 * wscale))}
        ent["verify"]["algorithmic_bytes"] = rec["verify_algorithmic_bytes"]
        if "fused" in ent:
            ent["fused"]["algorithmic_bytes"] = rec["roofline"]["algorithmic_bytes"]
        key = f"{rec['config']['workload_key']}:{rec['config']['solver']}:{rec['config']['waves']}"
        out["workloads"][key] = ent
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(out, indent=1, sort_keys=True))
    return 0


def run_solver_sweep(args):
    """Verify µs per solver on level trees (root, then levels of W nodes) over T, W and B: the
    table behind the AUTO dispatch. One JSON line per (T, W, B) cell with every solver's time
    and the kernel AUTO ran; ``--out`` appends the lines to a file."""
    import numpy as np
    import torch
    import synth
    import tree_speculative_verification_amd as tsv
    tsv.load()
    cells = []
    for T in (24, 32, 48, 64, 128, 256):
        for W in (1, 2, 4, 8, 16, 32, 64):
            if W < T:
                cells.append((T, W))
    lines = []
    for T, W in cells:
        par = synth.level_tree(T, W)
        depth = int(synth.tree_depths(par).max())
        for B in args.batches:
            inp = synth.make_inputs(B, 32, T, dtype="bf16", seed=7, parents=par)
            d = to_device(inp)
            res = {}
            solvers = ("auto", "fwdsub", "neumann", "level") if T > 64 else ("auto", "fwdsub", "neumann")
            for sv in solvers:
                fn = lambda: tsv.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                             d["parent"], solver=sv)
                fn()
                torch.cuda.synchronize()
                g = graph_of(fn, args.steps)
                res[sv] = round(min(time_graph(g, args.steps) for _ in range(2)), 3)
                del g
            best = min((v, k) for k, v in res.items() if k != "auto")[1]
            line = dict(T=T, W=W, depth=depth, B=B, H=32, us=res, best=best,
                        auto_kernel=verify_kernel_name(T, "auto", B * 32, 0, "bf16"))
            print(json.dumps(line), flush=True)
            lines.append(line)
    if args.out:
        with open(args.out, "a") as fh:
            for line in lines:
                fh.write(json.dumps(line) + "\n")
    return 0


def run_depth_sweep(args):
    """The solve strategies across tree depths 1-255 at T = 256 (level trees: a root, then
    levels of W nodes, depth ceil(255 / W)): verify µs at each of --batches. Solvers: AUTO
    (forward substitution in the fused kernels), NEUMANN (per 64-node block in the blocked
    kernel), the whole-tree series, its squaring form and the split design. One JSON line per
    (depth, B); ``--out`` appends them to a file. (Their bf16 errors against the oracle on the
    same trees are a GPU test: test_gpu_matrix_solvers.py::test_errors_by_depth.)"""
    import torch
    import synth
    import tree_speculative_verification_amd as tsv
    tsv.load()
    T = 256
    solvers = ("auto", "neumann", "series", "squaring", "split")
    lines = []
    for W in (255, 128, 64, 32, 16, 8, 4, 2, 1):
        par = synth.level_tree(T, W)
        depth = int(synth.tree_depths(par).max())
        for B in args.batches:
            inp = synth.make_inputs(B, 32, T, dtype="bf16", seed=11, parents=par)
            d = to_device(inp)
            res = {}
            for sv in solvers:
                ws = None
                if sv in tsv.WORKSPACE_SOLVERS:
                    ws = torch.empty((tsv.workspace_bytes(B, 32, T, sv),), dtype=torch.uint8, device="cuda")
                O = torch.empty((B, T, 32, 128), device="cuda")
                U = torch.empty_like(O)
                L = torch.empty((B, T, 32), device="cuda")
                fn = lambda: tsv.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                             d["parent"], solver=sv, out=(O, U, L), workspace=ws)
                fn()
                torch.cuda.synchronize()
                n = max(3, min(args.steps, 20))
                g = graph_of(fn, n)
                res[sv] = round(min(time_graph(g, n) for _ in range(2)), 3)
                del g, ws, O, U, L
            line = dict(T=T, W=W, depth=depth, B=B, H=32, us=res,
                        best=min((v, k) for k, v in res.items())[1])
            print(json.dumps(line), flush=True)
            lines.append(line)
    if args.out:
        with open(args.out, "a") as fh:
            for line in lines:
                fh.write(json.dumps(line) + "\n")
    return 0


def run_conv(args):
    """The root-path causal convolution (kernel 4, SiLU) and its state commit on the workload's
    trees, over the channels a GDN layer convolves: q and k of its q/k heads and v of its value
    heads (2 * 16 * 128 + 32 * 128 = 8192 for the 9B shape), bf16. One JSON line; HBM bytes
    per launch: x read and y written once per real node, plus the state, weights and parents."""
    import numpy as np
    import torch
    import tree_speculative_verification_amd as tsv
    wl = WORKLOADS[args.workload]
    B, T = wl["B"], wl["T"]
    C = 2 * 16 * 128 + 32 * 128
    K = 4
    inp = build_inputs(wl)
    g = torch.Generator(device="cpu").manual_seed(11)
    x = torch.randn((B, T, C), generator=g).to(torch.bfloat16).cuda()
    st = torch.randn((B, K - 1, C), generator=g).to(torch.bfloat16).cuda()
    w = (torch.randn((C, K), generator=g) * 0.5).cuda()
    d = to_device(inp)
    y = torch.empty_like(x)
    new = torch.empty_like(st)
    tsv.load()
    conv = lambda: tsv.tree_conv(x, w, st, d["parent"], silu=True, tree_len=d["tree_len"], out=y)
    commit = lambda: tsv.conv_commit(x, st, d["parent"], d["path"], d["path_len"],
                                     tree_len=d["tree_len"], out=new)
    for _ in range(args.warmup):
        conv()
        commit()
    torch.cuda.synchronize()
    gc = graph_of(conv, args.steps)
    us_conv = time_graph(gc, args.steps)
    del gc
    gm = graph_of(commit, args.steps)
    us_commit = time_graph(gm, args.steps)
    del gm
    lens = inp["tree_len"] if inp.get("tree_len") is not None else np.full(B, T)
    nodes = int(lens.sum())
    cbytes = 2 * nodes * C * 2 + B * (K - 1) * C * 2 + C * K * 4 + B * T * 4
    out = {"op": "tree_conv (K=4, SiLU) + conv_commit", "workload": wl["desc"],
           "workload_key": args.workload, "channels": C, "nodes": nodes, "dtype": "bf16",
           "conv_us": round(us_conv, 3), "conv_commit_us": round(us_commit, 3),
           "conv_bytes": cbytes, "conv_gbs": round(cbytes / (us_conv * 1e-6) / 1e9, 1),
           "conv_hbm_frac": round(cbytes / (us_conv * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "steps": args.steps, "launch": "hip graph of all timed launches"}
    print(json.dumps(out), flush=True)
    return 0


def build_inputs(wl):
    import numpy as np
    import synth
    kw = {k: wl[k] for k in ("B", "H", "T", "tree", "dtype", "seed")}
    lens = None
    if wl.get("ragged"):
        lo, hi = wl["ragged"]
        lens = np.random.default_rng(wl["seed"] + 7919).integers(lo, hi + 1, wl["B"]).astype(np.int32)
    return synth.make_inputs(tree_kw=wl.get("tree_kw"), HK=wl.get("HK"), tree_len=lens, **kw)


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
    tl = inp.get("tree_len")
    out["tree_len"] = None if tl is None else torch.from_numpy(tl.astype(np.int32)).cuda()
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


SETTLE_MS = 30.0  # untimed GPU time before a timed replay


def time_graph(g, n, settle_ms=SETTLE_MS):
    """Average µs per call of a graph of n calls: untimed replays until ``settle_ms`` of GPU time
    has run (at least one), then one replay between two events on the stream the replay runs
    on, synchronised on both sides. The GPU's clocks take about 15 ms of sustained work to
    settle: successive replays of a 3.3 ms graph (200 decode steps at B=16, T=16) ran 18.7,
    17.0, 16.6 and then 16.3 µs per step, and of a 2 ms graph of B=16, T=256 verifies 119 down to
    99 µs per call; a single warm replay left the timed one on a partly ramped GPU."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    spent, reps = 0.0, 0
    while reps < 1 or (spent < settle_ms and reps < 1000):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
        reps += 1
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
    plain = inp.get("tree_len") is None and inp.get("HK", inp["H"]) == inp["H"]
    while True:
        t0 = time.perf_counter()
        if plain:
            oracle.gdn_tree(inp["parent"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                            inp["S0"])
            oracle.commit(inp["parent"], inp["path"], inp["path_len"], inp["k"], inp["v"],
                          inp["alpha"], inp["beta"], inp["S0"])
        else:
            oracle.gdn_tree_ragged(inp["parent"], inp["tree_len"], inp["q"], inp["k"], inp["v"],
                                   inp["alpha"], inp["beta"], inp["S0"])
            oracle.commit_ragged(inp["parent"], inp["tree_len"], inp["path"], inp["path_len"],
                                 inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s and len(times) >= 3:
            break
        if len(times) >= 1 and times[0] > budget_s:
            break
    times.sort()
    med = times[len(times) // 2]
    return dict(value=med * 1e6, unit="us per layer (verify + commit)", cores=oracle.num_threads(),
                kind="oracle", sample=f"{len(times)} full layers of this workload, median")


def cpu_baseline_threads(inp, wl, reps=5):
    """The CPU baseline of the timing protocol: the oracle's wall time per layer (µs), median of
    `reps`, on every host core and on one.
    Large workloads run a slice of whole (sequence, head) problems, as many heads of sequence 0
    as there are threads (all cores) or 2 heads (one core), scaled by the number of such
    problems in the layer; every (sequence, head) problem costs the same up to its tree."""
    import oracle
    all_threads = oracle.num_threads()
    B, H = wl["B"], wl["H"]
    res = {}
    for label, threads in (("all_cores", all_threads), ("one_core", 1)):
        oracle.set_threads(threads)
        full = B * H * wl["T"] <= 2048
        hs = H if full else min(H, max(2, threads))
        if full:
            sub = dict(inp)
            scale = 1.0
        else:
            sub = {n: inp[n][:1, :, :hs] for n in ("q", "k", "v", "alpha", "beta")}
            sub["S0"] = inp["S0"][:1, :hs]
            for n in ("parent", "path"):
                sub[n] = inp[n][:1]
            sub["path_len"] = inp["path_len"][:1]
            scale = (B * H) / hs
        times = []
        for rep in range(reps + 1):  # the first call (thread team start-up) is not timed
            t0 = time.perf_counter()
            oracle.gdn_tree(sub["parent"], sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"], sub["S0"])
            oracle.commit(sub["parent"], sub["path"], sub["path_len"], sub["k"], sub["v"], sub["alpha"],
                          sub["beta"], sub["S0"])
            if rep:
                times.append((time.perf_counter() - t0) * scale)
        times.sort()
        res[label] = {"us_per_layer": round(times[len(times) // 2] * 1e6, 1), "threads": threads,
                      "sample": "whole layer" if full else f"sequence 0, {hs} heads, scaled x{scale:g}"}
    oracle.set_threads(all_threads)
    return res


# The workloads of the timing protocol: every configuration of the pages' workload table that
# fits one GPU, small and large batch.
PROTOCOL_WORKLOADS = ["binary7_fp32", "topk16_b1", "skewed64_b1", "skewed64_b16", "random256_b1",
                      "random256_b16"]


def environment():
    """Software versions, for the record of a measurement."""
    import subprocess
    import torch
    env = {"torch": torch.__version__, "hip_runtime": torch.version.hip, "rocm": None, "hipcc": None,
           "gpu": torch.cuda.get_device_name(0)}
    try:
        with open("/opt/rocm/.info/version") as fh:
            env["rocm"] = fh.read().strip()
    except OSError:
        pass
    try:
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True, text=True, timeout=60)
        env["hipcc"] = next((ln.strip() for ln in r.stdout.splitlines() if "version" in ln.lower()), None)
    except (OSError, subprocess.SubprocessError):
        pass
    return env


def gpu_state():
    """Clocks, temperature and power of GPU 0 as amd-smi reports them (None if unavailable)."""
    import subprocess
    for cmd in (["amd-smi", "metric", "-g", "0", "--json"], ["/opt/rocm/bin/amd-smi", "metric", "-g", "0", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=60)
        except (OSError, subprocess.SubprocessError):
            continue
        if r.returncode != 0:
            continue
        try:
            data = json.loads(r.stdout)
        except ValueError:
            return {"raw": r.stdout[:2000]}
        gpu = data[0] if isinstance(data, list) and data else data
        if isinstance(gpu, dict) and "gpu_data" in gpu:
            gpu = gpu["gpu_data"][0] if gpu["gpu_data"] else gpu
        if isinstance(gpu, dict):
            return {k: gpu[k] for k in ("clock", "temperature", "power") if k in gpu} or {"keys": sorted(gpu)[:40]}
        return {"raw": r.stdout[:2000]}
    return None


def _stats(xs):
    import numpy as np
    xs = np.asarray(xs, dtype=np.float64)
    return {"median_us": round(float(np.median(xs)), 3), "p10_us": round(float(np.percentile(xs, 10)), 3),
            "p90_us": round(float(np.percentile(xs, 90)), 3), "n": int(xs.size)}


def run_protocol(args):
    """Timing distributions per kernel (verify, commit, and the serial and hybrid verifies):
      warm  a HIP graph of back-to-back calls (--steps, a quarter of them for the serial and
            hybrid kernels) replayed 10 times with events around each replay: median, p10 and
            p90 of the per-call average over the replays (stream time);
      cold  --warmup + --steps eager rounds in which every call is preceded by a fill kernel
            writing 512 MiB (evicting L2 and the Infinity Cache), outside the events around the
            call, the compared kernels interleaved call by call: median, p10 and p90 of the
            per-call stream time (which includes the launch gap of an eager call).
    Run under rocprofv3 --kernel-trace, the same run gives per-dispatch device times, warm and
    cold apart (--protocol-summary). Also reports the oracle on all host cores and on one,
    software versions, and the GPU's clocks, temperature and power before and after."""
    import torch
    import tree_speculative_verification_amd as tsv
    tsv.load()
    names = args.protocol_workloads or PROTOCOL_WORKLOADS
    out = open(args.out, "a") if args.out else None
    flush = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
    for name in names:
        wl = WORKLOADS[name]
        B, H, T = wl["B"], wl["H"], wl["T"]
        inp = build_inputs(wl)
        d = to_device(inp)
        O = torch.empty((B, T, H, 128), device="cuda")
        U = torch.empty_like(O)
        ell = torch.empty((B, T, H), device="cuda")
        S_new = torch.empty_like(d["S0"])
        snaps = torch.empty((B, T, H, 128, 128), device="cuda")
        calls = {
            "verify": lambda: tsv.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                              d["parent"], out=(O, U, ell)),
            "commit": lambda: tsv.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"],
                                         d["path_len"], out=S_new),
            "serial_verify": lambda: tsv.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                       d["S0"], d["parent"], snapshots=snaps),
            "hybrid_verify": lambda: tsv.hybrid_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                       d["S0"], d["parent"], snapshots=snaps),
        }
        state_before = gpu_state()
        calls["verify"]()  # U for the commit
        torch.cuda.synchronize()
        warm = {}
        for k, fn in calls.items():
            n = args.steps if k in ("verify", "commit") else max(10, args.steps // 4)
            g = graph_of(fn, n)
            g.replay()
            torch.cuda.synchronize()
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(10)]
            for e0, e1 in pairs:
                e0.record()
                g.replay()
                e1.record()
            torch.cuda.synchronize()
            warm[k] = _stats([a.elapsed_time(b) * 1000.0 / n for a, b in pairs])
            warm[k]["calls_per_replay"] = n
            del g
        print(f"[protocol] {name}: warm done", file=sys.stderr, flush=True)
        n = args.steps + args.warmup
        ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(n)] for k in calls}
        for it in range(n):
            for k, fn in calls.items():
                flush.fill_(float(it))
                e0, e1 = ev[k][it]
                e0.record()
                fn()
                e1.record()
            if it % 25 == 24:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        cold = {k: _stats([a.elapsed_time(b) * 1000.0 for a, b in pairs[args.warmup:]])
                for k, pairs in ev.items()}
        print(f"[protocol] {name}: cold done", file=sys.stderr, flush=True)
        state_after = gpu_state()
        del snaps
        torch.cuda.empty_cache()
        rec = {"workload": name, "desc": wl["desc"], "steps": args.steps, "warmup": args.warmup,
               "stream_time": {"warm": warm, "cold": cold},
               "oracle": cpu_baseline_threads(inp, wl), "kernel_digest": kernel_digest(),
               "gpu_state_before": state_before, "gpu_state_after": state_after}
        if name == names[0]:
            rec["environment"] = environment()
        line = json.dumps(rec)
        print(line, flush=True)
        if out:
            out.write(line + "\n")
            out.flush()
    if out:
        out.close()
    return 0


def protocol_summary(trace_csv, warmup=25):
    """Per-dispatch device times from a rocprofv3 kernel trace of a --protocol run of one
    workload: each library kernel's dispatches split into cold (the dispatch right before it
    was the 512 MiB float fill) and warm (the rest), the first `warmup` cold ones of each kernel
    dropped; median, p10 and p90 of end - start."""
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out, prev = {}, ""
    for r in rows:
        name = r["Kernel_Name"]
        if "canopy::" in name:
            short = name.split("canopy::")[1].split("(")[0].split("<")[0]
            phase = "cold" if "FillFunctor<float>" in prev else "warm"
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            out.setdefault(phase, {}).setdefault(short, []).append(dur)
        prev = name
    for k in out.get("cold", {}):
        out["cold"][k] = out["cold"][k][warmup:]
    return {ph: {k: _stats(v) for k, v in ks.items()} for ph, ks in out.items()}


def trace_summary(trace_csv):
    """Device time per dispatch of each library kernel in a rocprofv3 kernel trace (end - start,
    µs): calls, average, median and minimum, keyed by the kernel's name with its template
    arguments (the profiles' kernel-trace tables)."""
    acc = {}
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"]
            if "canopy::" not in name:
                continue
            short = name.split("canopy::", 1)[1].split("(")[0]
            acc.setdefault(short, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    out = {}
    for k, v in acc.items():
        v = sorted(v)
        n = len(v)
        med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
        out[k] = {"calls": n, "average_us": round(sum(v) / n, 3), "median_us": round(med, 3),
                  "min_us": round(v[0], 3)}
    return out


def run_peaks(args):
    """Measured references for the roofline fractions: HBM bandwidth of a large device copy
    (read + write) and of a large reduction (read), dense MFMA throughput of a large bf16 and
    fp32 library GEMM (hipBLASLt through torch.matmul), and the time of an empty graph-replayed
    launch (a one-element fill), the floor of any single-launch step."""
    import torch
    res = {}

    def ev_time(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1000.0 / reps  # seconds per call

    n = 2 ** 31 // 4  # 2 GiB of fp32
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    t = ev_time(lambda: b.copy_(a), 20)
    res["hbm_copy_gbs"] = round(2 * a.numel() * 4 / t / 1e9, 1)
    t = ev_time(lambda: a.sum(), 20)
    res["hbm_read_gbs"] = round(a.numel() * 4 / t / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    for name, dt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
        m = 8192
        x = torch.randn(m, m, device="cuda").to(dt)
        y = torch.randn(m, m, device="cuda").to(dt)
        t = ev_time(lambda: torch.matmul(x, y), 10)
        res[f"gemm_{name}_tflops"] = round(2 * m ** 3 / t / 1e12, 1)
        del x, y
    torch.cuda.empty_cache()
    z = torch.empty(1, device="cuda")
    g = graph_of(lambda: z.fill_(0.0), 200)
    res["empty_launch_us"] = round(time_graph(g, 200), 3)
    res["notes"] = ("copy counts read + write bytes; GEMMs are 8192^3 through torch.matmul; the empty "
                    "launch is a one-element fill replayed 200 times in one graph")
    res["environment"] = environment()
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(line + "\n")
    return 0


def crossover_cpu_baseline(B, H, T, W, L, budget_s):
    """The oracle for one crossover round of a cell: one layer of the cell's shape (seeded
    synthetic inputs on its level tree) timed by cpu_baseline, scaled to the round's L layers
    (the layers are independent and cost the same) and to 100 rounds."""
    import synth
    inp = synth.make_inputs(B, H, T, dtype="bf16", seed=1000 * B + T * 17 + W, parents=synth.level_tree(T, W))
    cb = cpu_baseline(inp, budget_s)
    per_layer = cb["value"]
    return dict(value=round(per_layer * L, 1), unit=f"us per round ({L} layers, verify + commit)",
                per_layer_us=round(per_layer, 1), extrapolated_100_rounds_s=round(per_layer * L * 100 / 1e6, 2),
                cores=cb["cores"], kind="oracle",
                sample=f"one layer timed ({cb['sample']}), scaled to {L} layers and to 100 rounds")


def crossover_cells():
    """Depth x width level trees: root, then levels of W nodes (the last one partial);
    W = 1 is a chain; shapes that coincide (stars) are kept once; depth 1..64."""
    import synth
    seen, cells = set(), []
    for W in (1, 2, 4, 8, 16):
        for T in (3, 8, 16, 32, 64, 128, 256):
            par = synth.level_tree(T, W)
            D = int(synth.tree_depths(par).max())
            if not 1 <= D <= 64:
                continue
            key = tuple(par.tolist())
            if key in seen:
                continue
            seen.add(key)
            cells.append((W, T, D))
    return cells


def run_crossover(args):
    """24 stacked GDN layers, rounds of verify + commit that chain each layer's committed
    state, for every depth x width cell and batch size: the parallel path (24 tree verifies,
    then one launch committing all 24 layers), the chain hybrid (the same with the hybrid's
    verify) and the serial fork baseline (serial verify + snapshot commit per layer: committing
    all layers at once would keep 24 layers of per-node snapshots, 206 GB at B = 16, T = 256).
    One round (24 layers) is captured as a HIP graph; the accepted path of every round is copied
    in before its replay."""
    import numpy as np
    import torch
    import synth
    import tree_speculative_verification_amd as tsv
    tsv.load()
    L, H = 24, 32
    out = open(args.out, "a") if args.out else None
    gen = torch.Generator(device="cuda")
    for B in args.batches:
        for (W, T, D) in crossover_cells():
            if args.max_t and T > args.max_t:
                continue
            gen.manual_seed(1000 * B + T * 17 + W)
            par_np = synth.level_tree(T, W)
            parent = torch.from_numpy(np.broadcast_to(par_np, (B, T)).copy()).cuda()
            q, k, v, al, be, S0 = [], [], [], [], [], []
            for _ in range(L):
                xq = torch.randn(B, T, H, 128, device="cuda", generator=gen)
                xk = torch.randn(B, T, H, 128, device="cuda", generator=gen)
                q.append((xq / xq.norm(dim=-1, keepdim=True)).to(torch.bfloat16))
                k.append((xk / xk.norm(dim=-1, keepdim=True)).to(torch.bfloat16))
                v.append(torch.randn(B, T, H, 128, device="cuda", generator=gen).to(torch.bfloat16))
                be.append(torch.sigmoid(torch.randn(B, T, H, device="cuda", generator=gen)))
                al.append(torch.exp(-torch.nn.functional.softplus(torch.randn(B, T, H, device="cuda", generator=gen))))
                S0.append(0.1 * torch.randn(B, H, 128, 128, device="cuda", generator=gen))
            rng = np.random.default_rng(B * 7919 + T * 31 + W)
            R = args.rounds
            paths = np.full((R, B, T), -1, np.int32)
            plens = np.zeros((R, B), np.int32)
            for r in range(R):
                for b in range(B):
                    pth = synth.random_leaf_path(par_np, rng)
                    paths[r, b, :len(pth)] = pth
                    plens[r, b] = len(pth)
            paths_d = torch.from_numpy(paths).cuda()
            plens_d = torch.from_numpy(plens).cuda()
            path_cur = torch.empty((B, T), dtype=torch.int32, device="cuda")
            plen_cur = torch.empty((B,), dtype=torch.int32, device="cuda")
            O = torch.empty((B, T, H, 128), device="cuda")
            Us = [torch.empty_like(O) for _ in range(L)]  # every layer's U, for the one commit
            ell = torch.empty((B, T, H), device="cuda")
            S_par = [s.clone() for s in S0]
            S_ser = [s.clone() for s in S0]
            S_hyb = [s.clone() for s in S0]
            snaps = torch.empty((B, T, H, 128, 128), device="cuda")

            def round_parallel():
                # every layer verifies, then one launch commits the accepted path in all of them
                for l in range(L):
                    tsv.tree_verify(q[l], k[l], v[l], al[l], be[l], S_par[l], parent, out=(O, Us[l], ell))
                tsv.commit_layers(S_par, k, Us, al, parent, path_cur, plen_cur, outs=S_par)

            def round_serial():
                for l in range(L):
                    tsv.serial_verify(q[l], k[l], v[l], al[l], be[l], S_ser[l], parent, snapshots=snaps)
                    tsv.serial_commit(snaps, S_ser[l], parent, path_cur, plen_cur, out=S_ser[l])

            def round_hybrid():
                Uh = []
                for l in range(L):
                    Uh.append(tsv.hybrid_verify(q[l], k[l], v[l], al[l], be[l], S_hyb[l], parent,
                                                snapshots=snaps)[1])
                tsv.commit_layers(S_hyb, k, Uh, al, parent, path_cur, plen_cur, outs=S_hyb)

            def timed(fn, r0, rounds):
                """Rounds r0 .. r0+rounds-1 of the chain (each with its own accepted path)."""
                path_cur.copy_(paths_d[r0]); plen_cur.copy_(plens_d[r0])
                g = torch.cuda.CUDAGraph()
                torch.cuda.synchronize()
                with torch.cuda.graph(g):
                    fn()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for r in range(r0, r0 + rounds):
                    path_cur.copy_(paths_d[r]); plen_cur.copy_(plens_d[r])
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                del g
                return e0.elapsed_time(e1) * 1000.0 / rounds

            # Both sides start from the same states and commit the same path in round r. The
            # serial side times its first round alone, to size its run to the time budget.
            us_par = timed(round_parallel, 0, R)
            us_ser_probe = timed(round_serial, 0, 1)
            R_ser = int(max(0, min(R - 1, args.serial_budget * 1e6 / max(us_ser_probe, 1.0))))
            us_ser = timed(round_serial, 1, R_ser) if R_ser >= 1 else us_ser_probe
            rounds_ser = 1 + R_ser
            us_hyb_probe = timed(round_hybrid, 0, 1)
            R_hyb = int(max(0, min(R - 1, args.serial_budget * 1e6 / max(us_hyb_probe, 1.0))))
            us_hyb = timed(round_hybrid, 1, R_hyb) if R_hyb >= 1 else us_hyb_probe
            rounds_hyb = 1 + R_hyb

            def rel(xs, ys):
                return max(float((a - b).abs().max()) / max(float(b.abs().max()), 1e-30) for a, b in zip(xs, ys))
            err = rel(S_par, S_ser) if rounds_ser == R else None
            err_h = rel(S_par, S_hyb) if rounds_hyb == R else None
            rec = {"W": W, "T": T, "depth": D, "B": B, "H": H, "layers": L,
                   "rounds_parallel": R, "rounds_serial": rounds_ser,
                   "us_per_round_parallel": round(us_par, 2), "us_per_round_serial": round(us_ser, 2),
                   "us_per_layer_parallel": round(us_par / L, 3), "us_per_layer_serial": round(us_ser / L, 3),
                   "speedup_parallel_over_serial": round(us_ser / us_par, 3),
                   "final_state_rel_err_parallel_vs_serial": err,
                   "rounds_hybrid": rounds_hyb, "us_per_layer_hybrid": round(us_hyb / L, 3),
                   "speedup_parallel_over_hybrid": round(us_hyb / us_par, 3),
                   "speedup_hybrid_over_serial": round(us_ser / us_hyb, 3),
                   "final_state_rel_err_parallel_vs_hybrid": err_h}
            smallest = B == min(args.batches) and (W, T) == crossover_cells()[0][:2]
            largest = B == max(args.batches) and (W, T) == (16, 256)
            if not args.no_cpu and (smallest or largest):
                cb = crossover_cpu_baseline(B, H, T, W, L, args.cpu_budget)
                cb["speedup_parallel_over_oracle"] = round(cb["value"] / us_par, 1)
                rec["cpu_baseline"] = cb
            line = json.dumps(rec)
            print(line, flush=True)
            if out:
                out.write(line + "\n")
                out.flush()
            del q, k, v, al, be, S0, S_par, S_ser, S_hyb, snaps, O, Us
            torch.cuda.empty_cache()
    if out:
        out.close()
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-extra", action="store_true",
                    help="the default workload only (without the B=16 workloads beside it)")
    ap.add_argument("--solver", default="auto",
                    choices=["auto", "fwdsub", "neumann", "level", "series", "squaring", "split", "levelsync"])
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-serial", action="store_true", help="skip the serial fork baseline")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying a HIP graph")
    ap.add_argument("--crossover", action="store_true",
                    help="run the depth x width crossover over 24 layers instead of one workload")
    ap.add_argument("--rounds", type=int, default=100, help="crossover: rounds per cell")
    ap.add_argument("--solver-sweep", action="store_true",
                    help="time every solver on level trees over T, width and --batches")
    ap.add_argument("--depth-sweep", action="store_true",
                    help="time every solve strategy over tree depths 1-255 at T=256")
    ap.add_argument("--conv", action="store_true",
                    help="time the root-path causal convolution and its commit instead")
    ap.add_argument("--protocol", action="store_true",
                    help="per-call timing distributions (median, p10, p90), warm and cold, with "
                         "the oracle on all cores and one, versions and GPU clocks")
    ap.add_argument("--protocol-workloads", nargs="+", default=None, choices=sorted(WORKLOADS))
    ap.add_argument("--peaks", action="store_true",
                    help="measured HBM, GEMM and launch references for the roofline fractions")
    ap.add_argument("--trace-summary", default="", metavar="CSV",
                    help="per-kernel device time per dispatch from a rocprofv3 kernel trace CSV")
    ap.add_argument("--protocol-summary", default="", metavar="CSV",
                    help="device-time distributions from the rocprofv3 kernel trace CSV of a "
                         "--protocol run (no GPU work)")
    ap.add_argument("--batches", type=int, nargs="+", default=[1, 4, 16], help="crossover: batch sizes")
    ap.add_argument("--max-t", type=int, default=0, help="crossover: skip trees larger than this")
    ap.add_argument("--serial-budget", type=float, default=2.0,
                    help="crossover: seconds of serial rounds per cell (at most --rounds)")
    ap.add_argument("--out", default="", help="crossover: append JSON lines to this file")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="also run one plain device-to-device copy of this many bytes (a known "
                         "traffic reference for hardware counters)")
    ap.add_argument("--pmc-summary", default="", metavar="DIR",
                    help="summarise rocprofv3 --pmc runs found in DIR into the HBM traffic file "
                         "(no GPU work)")
    args = ap.parse_args(argv)
    if args.pmc_summary:
        return pmc_summary(args.pmc_summary, args.out or TRAFFIC_FILE)
    if args.protocol_summary:
        print(json.dumps(protocol_summary(args.protocol_summary)), flush=True)
        return 0
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary), indent=1, sort_keys=True), flush=True)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify and commit kernels shard by (sequence, "
              "head) with no exchange, and this benchmark measures one MI355X. Use --gpus 1.",
              file=sys.stderr)
        return 2
    if args.crossover:
        return run_crossover(args)
    if args.conv:
        return run_conv(args)
    if args.solver_sweep:
        return run_solver_sweep(args)
    if args.depth_sweep:
        return run_depth_sweep(args)
    if args.protocol:
        return run_protocol(args)
    if args.peaks:
        return run_peaks(args)

    rec = measure(args.workload, args, baselines=not args.no_serial)
    primary = args.workload == DEFAULT_WORKLOAD and not args.no_extra
    out = {
        "metric": METRIC,
        "value": rec["step_us"],
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["step_us"] / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec.pop("dtype"),
        "data": "synthetic",
    }
    out.update(rec)
    out["kernel_digest"] = kernel_digest()
    if primary:
        # The other workloads the targets name, timed the same way in the same run: the
        # 256-node trees at B=16 (the MFMA target's configuration) and 16-node trees at B=16
        # (the HBM target's tree size at a batch that can fill the GPU).
        out["extra_workloads"] = []
        for key in EXTRA_WORKLOADS:
            r = measure(key, args, baselines=False)
            r.pop("dtype")
            out["extra_workloads"].append(r)
    if primary:
        # The streaming copy rate of this GPU, measured in the same run: the practical HBM
        # ceiling next to the published 8 TB/s (each roofline also gives its share of it).
        out["copy_gbs"] = copy_rate_gbs()
        for r in [out] + out["extra_workloads"]:
            if r.get("roofline", {}).get("unit") == "GB/s":
                r["roofline"]["copy_frac"] = round(r["roofline"]["achieved"] / out["copy_gbs"], 4)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(build_inputs(WORKLOADS[args.workload]), args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


def copy_rate_gbs(nbytes=2 ** 31, reps=10):
    """Device-to-device copy of nbytes (fp32, far past the 256 MB Infinity Cache), bytes read
    plus written per second, in GB/s."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1000.0 / reps
    del a, b
    torch.cuda.empty_cache()
    return round(2 * nbytes / t / 1e9, 1)


def measure(key, args, baselines=True):
    """Time one workload's decode step (exactly args.steps steps after args.warmup), the same
    work as separate calls, verify and commit alone and, with ``baselines``, the serial fork and
    the chain hybrid; returns the record of the bench line for it."""
    import numpy as np
    import torch
    import tree_speculative_verification_amd as tsv

    wl = WORKLOADS[key]
    B, H, T, dt = wl["B"], wl["H"], wl["T"], wl["dtype"]
    inp = build_inputs(wl)
    d = to_device(inp)
    tsv.load()
    print(f"[bench] {key}: inputs resident", file=sys.stderr, flush=True)
    O = torch.empty((B, T, H, 128), device="cuda")
    U = torch.empty_like(O)
    ell = torch.empty((B, T, H), device="cuda")
    S_new = torch.empty_like(d["S0"])

    ws_solver = args.solver in tsv.WORKSPACE_SOLVERS
    ws = None
    if ws_solver:
        ws = torch.empty((max(tsv.workspace_bytes(B, H, T, args.solver), 16),), dtype=torch.uint8,
                         device="cuda")

    def verify():
        tsv.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                        solver=args.solver, waves=args.waves, out=(O, U, ell), tree_len=d["tree_len"],
                        workspace=ws)

    def commit():
        tsv.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"], out=S_new,
                   tree_len=d["tree_len"])

    def separate_step():
        verify()
        commit()

    # The decode loop's step: commit the previous round's path (its U from the previous step)
    # into the carried state S_run, then verify the tree from it; U is carried in one buffer.
    S_run = d["S0"].clone()
    O_run = torch.empty_like(O)
    U_run = torch.empty_like(O)
    ell_run = torch.empty_like(ell)

    def step():
        if ws_solver:
            # the matrix forms: the commit, then the verify from the committed state
            tsv.commit(S_run, d["k"], U_run, d["alpha"], d["parent"], d["path"], d["path_len"],
                       out=S_run, tree_len=d["tree_len"])
            tsv.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_run, d["parent"],
                            solver=args.solver, out=(O_run, U_run, ell_run), tree_len=d["tree_len"],
                            workspace=ws)
            return
        tsv.commit_verify(S_run, d["k"], U_run, d["alpha"], d["parent"], d["path"], d["path_len"],
                          d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["parent"],
                          solver=args.solver, waves=args.waves, out=(O_run, U_run, ell_run),
                          S_out=S_run, tree_len_prev=d["tree_len"], tree_len=d["tree_len"])

    for _ in range(args.warmup):
        separate_step()
    torch.cuda.synchronize()
    ref_O, ref_U, ref_S = O.clone(), U.clone(), S_new.clone()
    tsv.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_run, d["parent"],
                    solver=args.solver, waves=args.waves, out=(O_run, U_run, ell_run),
                    tree_len=d["tree_len"], workspace=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.eager:
        us_step = time_eager(step, args.steps, 0)
        us_sep = time_eager(separate_step, args.steps, 0)
        us_verify = time_eager(verify, args.steps, 5)
        us_commit = time_eager(commit, args.steps, 5)
    else:
        # Timed region: one replay of a graph holding exactly `steps` steps. The loop carries
        # its state, so the replay is checked against the same steps run eagerly from the same
        # starting state, bit for bit.
        start = (S_run.clone(), U_run.clone())
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        eager_end = (S_run.clone(), U_run.clone(), O_run.clone())
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            for _ in range(args.steps):
                step()
        torch.cuda.synchronize()
        S_run.copy_(start[0])
        U_run.copy_(start[1])
        torch.cuda.synchronize()
        g_step.replay()
        torch.cuda.synchronize()
        if not (torch.equal(S_run, eager_end[0]) and torch.equal(U_run, eager_end[1])
                and torch.equal(O_run, eager_end[2])):
            raise RuntimeError("graph replay of the decode steps differs from the eager run")
        us_step = time_graph(g_step, args.steps)
        del g_step, start, eager_end
        g_sep = graph_of(separate_step, args.steps)
        us_sep = time_graph(g_sep, args.steps)
        # The replayed kernels must reproduce the eager results bit for bit.
        if not (torch.equal(O, ref_O) and torch.equal(U, ref_U) and torch.equal(S_new, ref_S)):
            raise RuntimeError("graph replay differs from the eager run")
        del g_sep
        g_v = graph_of(verify, args.steps)
        us_verify = time_graph(g_v, args.steps)
        del g_v
        g_c = graph_of(commit, args.steps)
        us_commit = time_graph(g_c, args.steps)
        del g_c
    if not bool(torch.isfinite(S_run).all()):
        raise RuntimeError("the carried state is not finite")
    us_serial = us_hybrid = None
    if baselines:
        snaps = torch.empty((B, T, H, 128, 128), device="cuda")

        def serial():
            tsv.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                              snapshots=snaps, tree_len=d["tree_len"])
        n_ser = max(10, args.steps // 4)
        if args.eager:
            us_serial = time_eager(serial, n_ser, 3)
        else:
            g_s = graph_of(serial, n_ser)
            us_serial = time_graph(g_s, n_ser)
            del g_s
        def hybrid():
            tsv.hybrid_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                              snapshots=snaps, tree_len=d["tree_len"])
        if args.eager:
            us_hybrid = time_eager(hybrid, n_ser, 3)
        else:
            g_h = graph_of(hybrid, n_ser)
            us_hybrid = time_graph(g_h, n_ser)
            del g_h
        del snaps

    if args.copy_probe:
        src = torch.empty(args.copy_probe // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] {key}: step {us_step:.3f} us", file=sys.stderr, flush=True)

    HK = wl.get("HK", H)
    lens = inp["tree_len"] if inp.get("tree_len") is not None else np.full(B, T)
    nodes = int(lens.sum())
    m_total = int(inp["path_len"].sum())
    vbytes = verify_bytes(B, H, T, dt, HK=HK, nodes=nodes)
    vflops = method_flops(inp["parent"], H, lens)
    vdense = verify_flops_ragged(H, lens)
    one = one_launch_step(T, args.solver, B * H, args.waves)
    if one:
        # the dominant (only) kernel of the step: commit + verify in one launch per step
        rbytes = fused_step_bytes(B, H, T, dt, m_total, HK=HK, nodes=nodes)
        rflops = vflops + commit_flops(H, m_total)
        rdense = vdense + commit_flops(H, m_total)
        r_us, r_kernel, r_role = us_step, fused_kernel_name(T, dt, B * H, args.waves), "fused"
        r_note = ("one launch per step (commit + verify): the method's flops of both, from the "
                  "trees' ancestor pairs and the accepted paths")
    else:
        rbytes, rflops, rdense, r_us, r_role = vbytes, vflops, vdense, us_verify, "verify"
        r_kernel = verify_kernel_name(T, args.solver, B * H, args.waves, dt)
        r_note = "the verify launch: the method's flops from the trees' ancestor pairs"
    achieved = rbytes / (r_us * 1e-6) / 1e9
    tflops = rflops / (r_us * 1e-6) / 1e12
    return {
        "dtype": "bf16" if dt == "bf16" else "fp32",
        "config": {"workload": wl["desc"], "workload_key": key, "B": B, "H": H, "T": T,
                   "q_k_heads": HK, "nodes": nodes, "dk": 128, "dv": 128, "tree": wl["tree"],
                   "solver": args.solver,
                   "waves": args.waves,
                   "step": ("commit of the previous round's accepted path (a random root-to-leaf "
                            "path) into the carried state, then verify of the tree from it "
                            "(canopy_commit_verify, %s)" % ("one launch" if one else "two launches")),
                   "launch": "eager" if args.eager else (
                       "hip graph of all timed steps, replayed untimed for at least %g ms of GPU "
                       "time before the one timed replay" % SETTLE_MS),
                   "copy_probe_bytes": args.copy_probe},
        "step_us": round(us_step, 3),
        "nodes_per_s": round(nodes / (us_step * 1e-6), 1),
        "separate_step_us": round(us_sep, 3),
        "verify_us": round(us_verify, 3),
        "verify_nodes_per_s": round(nodes / (us_verify * 1e-6), 1),
        "commit_us": round(us_commit, 3),
        "serial_verify_us": None if us_serial is None else round(us_serial, 3),
        "hybrid_verify_us": None if us_hybrid is None else round(us_hybrid, 3),
        "roofline": {"bound": "hbm", "kernel": r_kernel,
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": measured_traffic(key, args.solver, args.waves, r_role),
                     "algorithmic_bytes": rbytes, "launch_us": round(r_us, 3)},
        "verify_algorithmic_bytes": vbytes,
        "mfma": {"flops_per_launch": rflops, "achieved_tflops": round(tflops, 3),
                 "peak_tflops": BF16_PEAK_TFLOPS, "frac": round(tflops / BF16_PEAK_TFLOPS, 5),
                 "issued_dense_flops": rdense,
                 "issued_dense_frac": round(rdense / (r_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 5),
                 "note": r_note},
    }


if __name__ == "__main__":
    sys.exit(main())
