"""GPU parity: the HIP path through the C ABI against the oracle on the same seeded inputs.

Tolerances: max per-(batch, head) relative error (infinity norm) 2e-3 for bf16 q/k/v with fp32
state, 1e-5 for fp32 inputs; the ancestor mask, depth and statuses bit-exact; ell within
1e-5 * max(1, |ell|)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL, assert_close_heads, assert_close_state, assert_ell, oracle_commit,
                      report_metrics, run_oracle, slice_inputs, to_device)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


def _verify(canopy, d, **kw):
    import torch
    out = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                             d["parent"], structure=True, **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _check_structure(inp, mask, depth, status):
    dep_ref, mask_ref, st_ref = oracle.tree_structure(inp["parent"])
    assert np.array_equal(status, st_ref)
    assert np.array_equal(depth, dep_ref)
    assert np.array_equal(mask.view(np.uint32), mask_ref)


# ---------------------------------------------------------------------------------------------
def test_config_binary7_fp32(canopy):
    """The 7-node binary tree, fp32, B=1 H=2, seed 0; commit of path 0 -> 1 -> 3."""
    import torch
    inp = synth.make_inputs(1, 2, 7, tree="binary7", dtype="fp32", seed=0)
    inp["path"][:] = -1
    inp["path"][0, :3] = [0, 1, 3]
    inp["path_len"][:] = 3
    d = to_device(inp)
    ref = run_oracle(inp, accept=[3])
    for solver in ("fwdsub", "neumann", "level", "auto"):
        for waves in (1, 2, 4, 8):
            _say("binary7 fp32", solver, "waves", waves)
            O, U, ell, mask, depth, st = _verify(canopy, d, solver=solver, waves=waves)
            assert_close_heads("O", O, ref["O"], TOL["fp32"])
            assert_close_heads("U", U, ref["U"], TOL["fp32"])
            assert_ell(ell, ref["ell"])
            _check_structure(inp, mask, depth, st)
    _say("binary7 fp32 commit")
    O, U, ell = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
    Sn, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
    torch.cuda.synchronize()
    assert pst.cpu().numpy().tolist() == [0]
    assert_close_state("S_new", Sn.cpu().numpy(), ref["S_accept"], TOL["fp32"])
    S_or, _ = oracle_commit(inp)
    assert_close_state("S_new vs path recurrence", Sn.cpu().numpy(), S_or, TOL["fp32"])
    report_metrics("C1", "O", O.cpu().numpy(), ref["O"])
    report_metrics("C1", "U", U.cpu().numpy(), ref["U"])
    report_metrics("C1", "S_new", Sn.cpu().numpy(), S_or, state=True)


@pytest.mark.parametrize("solver", ["fwdsub", "neumann", "level", "auto"])
def test_config_topk16_bf16(canopy, solver):
    """The 1+3+12 top-k tree at the 9B layer's shape: B=1 H=32 T=16 bf16, commit of a random
    root-to-leaf path."""
    import torch
    inp = synth.make_inputs(1, 32, 16, tree="topk", tree_kw={"branching": (3, 4)}, dtype="bf16", seed=1)
    d = to_device(inp)
    ref = run_oracle(inp)
    _say("topk16 bf16", solver)
    O, U, ell, mask, depth, st = _verify(canopy, d, solver=solver)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    assert_ell(ell, ref["ell"])
    _check_structure(inp, mask, depth, st)
    Ut = torch.from_numpy(U).cuda()
    Sn, pst = canopy.commit(d["S0"], d["k"], Ut, d["alpha"], d["parent"], d["path"], d["path_len"])
    torch.cuda.synchronize()
    S_or, st_or = oracle_commit(inp)
    assert np.array_equal(pst.cpu().numpy(), st_or)
    assert_close_state("S_new", Sn.cpu().numpy(), S_or, TOL["bf16"])
    if solver == "auto":
        report_metrics("C2", "O", O, ref["O"])
        report_metrics("C2", "U", U, ref["U"])
        report_metrics("C2", "S_new", Sn.cpu().numpy(), S_or, state=True)


EDGE_T = [1, 2, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T", EDGE_T)
def test_tile_edges(canopy, T, dtype):
    """Every tile edge of the 16-row MFMA tiles and 64-node blocks, across tree families,
    solvers and workgroup widths."""
    kinds = ["random", "skewed", "chain", "star", "level"]
    kind = kinds[T % len(kinds)]
    kw = {"width": 3} if kind == "level" else {}
    inp = synth.make_inputs(2, 2, T, tree=kind, tree_kw=kw, dtype=dtype, seed=100 + T)
    d = to_device(inp)
    ref = run_oracle(inp)
    for solver, waves in (("fwdsub", 1), ("neumann", 2), ("level", 4), ("auto", 8), ("fwdsub", 8),
                          ("auto", 2), ("neumann", 4), ("fwdsub", 4), ("auto", 4)):
        _say("edge", T, dtype, kind, solver, waves)
        O, U, ell, mask, depth, st = _verify(canopy, d, solver=solver, waves=waves)
        assert_close_heads("O", O, ref["O"], TOL[dtype])
        assert_close_heads("U", U, ref["U"], TOL[dtype])
        assert_ell(ell, ref["ell"])
        _check_structure(inp, mask, depth, st)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
def test_config_skewed64_batch_sweep(canopy, B):
    """B in {1..16}, H=32, T=64 skewed trees (independent per sequence), bf16, every solver and
    the serial baseline; every (b, h) pair against the oracle (about 0.1 s of oracle at B=16 on
    16 host cores)."""
    import time
    import torch
    inp = synth.make_inputs(B, 32, 64, tree="skewed", dtype="bf16", seed=200 + B)
    d = to_device(inp)
    t0 = time.perf_counter()
    ref = run_oracle(inp)
    _say("skewed64 B", B, "oracle over the full grid: %.2f s" % (time.perf_counter() - t0))
    for solver in ("fwdsub", "neumann", "level", "auto"):
        _say("skewed64 B", B, solver)
        O, U, ell, mask, depth, st = _verify(canopy, d, solver=solver)
        assert_close_heads("O", O, ref["O"], TOL["bf16"])
        assert_close_heads("U", U, ref["U"], TOL["bf16"])
        assert_ell(ell, ref["ell"])
        _check_structure(inp, mask, depth, st)
    report_metrics(f"C3 B={B}", "O", O, ref["O"])
    report_metrics(f"C3 B={B}", "U", U, ref["U"])
    _say("skewed64 serial B", B)
    O, U, snap, st = canopy.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
    torch.cuda.synchronize()
    O, U = O.cpu().numpy(), U.cpu().numpy()
    del snap
    assert_close_heads("serial O", O, ref["O"], TOL["bf16"])
    assert_close_heads("serial U", U, ref["U"], TOL["bf16"])


def test_config_random256_b16(canopy):
    """The large tree at full size, in the launch configuration the benchmark uses: B=16 H=32
    T=256 random recursive trees, bf16; every (b, h) pair of verify (every solver) and commit of
    random leaves against the oracle (about 1 s of oracle on 16 host cores)."""
    import time
    import torch
    inp = synth.make_inputs(16, 32, 256, tree="random", dtype="bf16", seed=300)
    d = to_device(inp)
    t0 = time.perf_counter()
    ref = run_oracle(inp)
    _say("random256 B16 oracle over the full grid: %.2f s" % (time.perf_counter() - t0))
    for solver in ("fwdsub", "neumann", "level"):
        _say("random256 B16 verify", solver)
        O, U, ell, mask, depth, st = _verify(canopy, d, solver=solver)
        assert_close_heads("O", O, ref["O"], TOL["bf16"])
        assert_close_heads("U", U, ref["U"], TOL["bf16"])
    _say("random256 B16 verify auto")
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    assert_ell(ell, ref["ell"])
    _check_structure(inp, mask, depth, st)
    _say("random256 B16 commit")
    Sn, pst = canopy.commit(d["S0"], d["k"], torch.from_numpy(U).cuda(), d["alpha"], d["parent"],
                            d["path"], d["path_len"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    S_or, st_or = oracle_commit(inp)
    _say("random256 B16 oracle commit over the full grid: %.2f s" % (time.perf_counter() - t0))
    assert np.array_equal(pst.cpu().numpy(), st_or)
    assert_close_state("S_new", Sn.cpu().numpy(), S_or, TOL["bf16"])
    report_metrics("C4", "O", O, ref["O"])
    report_metrics("C4", "U", U, ref["U"])
    report_metrics("C4", "S_new", Sn.cpu().numpy(), S_or, state=True)


def test_serial_snapshots_match_oracle_states(canopy):
    import torch
    for dtype in ("fp32", "bf16"):
        inp = synth.make_inputs(2, 3, 40, tree="random", dtype=dtype, seed=400)
        d = to_device(inp)
        ref = run_oracle(inp, all_states=True)
        _say("serial snapshots", dtype)
        O, U, snap, st = canopy.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
        torch.cuda.synchronize()
        assert st.cpu().numpy().tolist() == [0, 0]
        assert_close_heads("serial O", O.cpu().numpy(), ref["O"], TOL[dtype])
        assert_close_heads("serial U", U.cpu().numpy(), ref["U"], TOL[dtype])
        sn = snap.cpu().numpy()  # [B,T,H,128,128]
        B, T, H = 2, 40, 3
        x = sn.reshape(B * T * H, 1, 128, 128)
        y = ref["S_all"].reshape(B * T * H, 1, 128, 128)
        assert_close_state("snapshots", x, y, TOL[dtype])


def test_serial_commit(canopy):
    """The serial baseline's commit copies the accepted node's snapshot: it equals the oracle's
    path recurrence; an empty path keeps S0; bad paths give their status and NaN."""
    import torch
    inp = synth.make_inputs(3, 2, 30, tree="skewed", dtype="bf16", seed=450)
    inp["path_len"][1] = 0
    d = to_device(inp)
    _say("serial verify + commit")
    O, U, snap, st = canopy.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
    Sn, pst = canopy.serial_commit(snap, d["S0"], d["parent"], d["path"], d["path_len"])
    torch.cuda.synchronize()
    S_or, st_or = oracle_commit(inp)
    assert pst.cpu().numpy().tolist() == st_or.tolist() == [0, 0, 0]
    assert torch.equal(Sn[1], d["S0"][1])
    assert_close_state("serial S_new", Sn.cpu().numpy(), S_or, TOL["bf16"])
    bad = d["path"].clone()
    bad[0, 1] = 30  # a node id out of range at position 1
    Sn2, pst2 = canopy.serial_commit(snap, d["S0"], d["parent"], bad, d["path_len"])
    torch.cuda.synchronize()
    assert pst2.cpu().numpy().tolist()[0] == 2
    assert torch.isnan(Sn2[0]).all()


def test_prep_entry_point(canopy):
    import torch
    for T in (1, 5, 33, 100, 256):
        inp = synth.make_inputs(3, 2, T, tree="skewed", dtype="fp32", seed=500 + T)
        d = to_device(inp)
        _say("prep", T)
        mask, depth, ell, st = canopy.tree_prep(d["parent"], d["alpha"])
        torch.cuda.synchronize()
        _check_structure(inp, mask.cpu().numpy(), depth.cpu().numpy(), st.cpu().numpy())
        ref = run_oracle(inp)
        assert_ell(ell.cpu().numpy(), ref["ell"])


def test_invalid_tree_and_path_reported(canopy):
    """A malformed tree gives its status and NaN outputs for that sequence only; malformed
    paths give their status and a NaN state; nothing blocks."""
    import torch
    inp = synth.make_inputs(3, 2, 20, tree="random", dtype="bf16", seed=600)
    inp["parent"][1, 7] = 9            # forward parent: node 7 is bad
    d = to_device(inp)
    _say("invalid tree")
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert st.tolist() == [0, 8, 0]
    assert np.isnan(O[1]).all() and np.isnan(U[1]).all() and np.isnan(ell[1]).all()
    assert np.isfinite(O[[0, 2]]).all() and np.isfinite(U[[0, 2]]).all()
    assert (mask[1] == 0).all() and (depth[1] == 0).all()
    _say("invalid tree serial")
    O2, U2, _, st2 = canopy.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
    torch.cuda.synchronize()
    assert st2.cpu().numpy().tolist() == [0, 8, 0]
    assert np.isnan(O2.cpu().numpy()[1]).all()

    inp = synth.make_inputs(4, 2, 7, tree="binary7", dtype="fp32", seed=601)
    paths = np.full((4, 7), -1, np.int32)
    paths[0, :3] = [0, 1, 3]      # valid
    paths[1, :3] = [0, 2, 3]      # 3 is not a child of 2 -> position 2
    paths[2, :2] = [1, 3]         # does not start at a root -> position 0
    plen = np.array([3, 3, 2, 9], np.int32)   # last: length out of range
    inp["path"], inp["path_len"] = paths, plen
    d = to_device(inp)
    _, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
    _say("invalid paths commit")
    Sn, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
    torch.cuda.synchronize()
    S_or, st_or = oracle_commit(inp)
    assert pst.cpu().numpy().tolist() == st_or.tolist() == [0, 3, 1, -1]
    Sn = Sn.cpu().numpy()
    assert np.isnan(Sn[1:]).all()
    assert_close_state("S_new", Sn[:1], S_or[:1], TOL["fp32"])


@pytest.mark.parametrize("kind,T", [("chain", 200), ("chain", 33), ("chain", 64), ("chain", 65),
                                    ("chain", 129), ("skewed", 128), ("random", 256)])
def test_commit_long_paths(canopy, kind, T):
    """Paths of many lengths up to T (chains commit all T nodes): the commit walks the path 64
    positions at a time, 4 at a time within those, so chains of 33, 64, 65, 129 and 200 nodes
    put the path's end on and just past every chunk edge."""
    import torch
    for dtype in ("bf16", "fp32"):
        inp = synth.make_inputs(4, 2, T, tree=kind, dtype=dtype, seed=900 + T)
        rng = np.random.default_rng(T)
        for b in range(4):  # accepted node anywhere on the tree, not only leaves
            a_node = int(rng.integers(0, T)) if b else T - 1
            pth = synth.root_path(inp["parent"][b], a_node)
            inp["path"][b] = -1
            inp["path"][b, :len(pth)] = pth
            inp["path_len"][b] = len(pth)
        d = to_device(inp)
        _say("commit long paths", kind, T, dtype, inp["path_len"].tolist())
        _, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
        Sn, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
        Sn2, _ = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
        torch.cuda.synchronize()
        assert torch.equal(Sn, Sn2)
        S_or, st_or = oracle_commit(inp)
        assert pst.cpu().numpy().tolist() == st_or.tolist() == [0, 0, 0, 0]
        assert_close_state("S_new", Sn.cpu().numpy(), S_or, TOL[dtype])


def test_commit_bad_link_in_a_later_chunk(canopy):
    """A path of 150 nodes on a chain whose 101st entry is not a child of the 100th: the check
    of the third 64-position chunk reports it, with the oracle's status code, and the state of
    that sequence is NaN while the other sequence commits normally."""
    import torch
    T = 160
    inp = synth.make_inputs(2, 2, T, tree="chain", dtype="bf16", seed=4242)
    for b in range(2):
        inp["path"][b] = -1
        inp["path"][b, :150] = np.arange(150)
        inp["path_len"][b] = 150
    inp["path"][1, 100] = 120
    d = to_device(inp)
    _, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
    Sn, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
    torch.cuda.synchronize()
    S_or, st_or = oracle_commit(inp)
    assert st_or[0] == 0 and st_or[1] > 0
    assert pst.cpu().numpy().tolist() == st_or.tolist()
    Sn = Sn.cpu().numpy()
    assert np.isnan(Sn[1]).all()
    assert_close_state("S_new", Sn[:1], S_or[:1], TOL["bf16"])


def test_commit_empty_path_and_in_place(canopy):
    import torch
    inp = synth.make_inputs(2, 4, 30, tree="skewed", dtype="bf16", seed=700)
    inp["path_len"][0] = 0
    d = to_device(inp)
    _, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
    _say("commit out-of-place")
    Sn, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
    S_copy = d["S0"].clone()
    _say("commit in place")
    Sn2, _ = canopy.commit(S_copy, d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"], out=S_copy)
    torch.cuda.synchronize()
    assert torch.equal(Sn, S_copy)
    assert torch.equal(Sn[0], d["S0"][0])  # empty path commits nothing
    S_or, _ = oracle_commit(inp)
    assert_close_state("S_new", Sn.cpu().numpy(), S_or, TOL["bf16"])


def test_hundred_rounds_chained_fp32(canopy):
    """Verify + commit for 100 rounds, each on a fresh random tree, feeding S_new into the next
    round. Equals one sequential recurrence over the concatenated accepted tokens: the oracle
    chains its own committed state; the page's tier-A bound is 1e-3 relative Frobenius after
    100 rounds (the per-round bound used here is the tighter 1e-4 infinity norm)."""
    import torch
    B, H, T = 2, 2, 12
    S_gpu = None
    S_ref = None
    worst = 0.0
    for rnd in range(100):
        inp = synth.make_inputs(B, H, T, tree="random", dtype="fp32", seed=10_000 + rnd)
        if S_ref is None:
            S_ref = inp["S0"].astype(np.float64)
        else:
            inp["S0"] = S_gpu.cpu().numpy()
        d = to_device(inp)
        if S_gpu is not None:
            d["S0"] = S_gpu
        if rnd % 25 == 0:
            _say("rounds", rnd)
        _, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])
        S_gpu, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
        ref_inp = dict(inp)
        ref_inp["S0"] = S_ref
        S_ref, _ = oracle_commit(ref_inp)
        Sg = S_gpu.cpu().numpy().astype(np.float64)
        fro = np.linalg.norm((Sg - S_ref).ravel()) / np.linalg.norm(S_ref.ravel())
        worst = max(worst, fro)
    assert worst <= 1e-3, worst


def test_deterministic_and_guarded(canopy):
    """Five runs are bitwise identical, inputs are untouched and no byte outside the outputs is
    written (canary guards around O, U and ell)."""
    import torch
    inp = synth.make_inputs(2, 4, 100, tree="random", dtype="bf16", seed=800)
    d = to_device(inp)
    before = {n: t.clone() for n, t in d.items()}
    B, T, H = 2, 100, 4
    n_o = B * T * H * 128
    guard = 4096
    bufO = torch.full((n_o + 2 * guard,), 1234.5, device="cuda")
    bufU = torch.full((n_o + 2 * guard,), -987.25, device="cuda")
    bufL = torch.full((B * T * H + 2 * guard,), 77.0, device="cuda")
    outs = []
    for rep in range(5):
        _say("determinism rep", rep)
        O = bufO[guard:guard + n_o].view(B, T, H, 128)
        U = bufU[guard:guard + n_o].view(B, T, H, 128)
        L = bufL[guard:guard + B * T * H].view(B, T, H)
        canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"], out=(O, U, L))
        torch.cuda.synchronize()
        outs.append((O.clone(), U.clone(), L.clone()))
    for o in outs[1:]:
        for x, y in zip(o, outs[0]):
            assert torch.equal(x, y)
    for buf, val in ((bufO, 1234.5), (bufU, -987.25), (bufL, 77.0)):
        assert bool((buf[:guard] == val).all()) and bool((buf[-guard:] == val).all())
    for n, t in d.items():
        assert torch.equal(t, before[n]), n


def test_host_errors(canopy):
    """Host-checkable errors return a status and launch nothing."""
    import ctypes
    import torch
    lib = canopy.load()
    inp = synth.make_inputs(1, 1, 4, tree="chain", dtype="fp32", seed=1)
    d = to_device(inp)
    O = torch.empty((1, 4, 1, 128), device="cuda")
    U = torch.empty_like(O)
    L = torch.empty((1, 4, 1), device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [p(d["q"]), p(d["k"]), p(d["v"]), p(d["alpha"]), p(d["beta"]), p(d["S0"]), p(d["parent"]),
            None]
    outs = [p(O), p(U), p(L), None, None, None]
    s = ctypes.c_void_p(0)
    # B, H, HV, T, dtype
    assert lib.canopy_tree_verify(*args, 1, 1, 1, 0, 0, *outs, 0, 0, s) == 1      # T = 0
    assert lib.canopy_tree_verify(*args, 1, 1, 1, 257, 0, *outs, 0, 0, s) == 1    # T > 256
    assert lib.canopy_tree_verify(*args, 1, 2, 1, 4, 0, *outs, 0, 0, s) == 1      # H > HV
    assert lib.canopy_tree_verify(*args, 1, 2, 3, 4, 0, *outs, 0, 0, s) == 1      # H does not divide HV
    assert lib.canopy_tree_verify(*args, 1, 0, 1, 4, 0, *outs, 0, 0, s) == 1      # H = 0
    assert lib.canopy_tree_verify(*args, 1, 1, 1, 4, 5, *outs, 0, 0, s) == 2      # dtype
    assert lib.canopy_tree_verify(*args, 1, 1, 1, 4, 0, *outs, 7, 0, s) == 2      # solver
    assert lib.canopy_tree_verify(*args, 1, 1, 1, 4, 0, *outs, 0, 3, s) == 2      # waves
    bad = list(args)
    bad[0] = None
    assert lib.canopy_tree_verify(*bad, 1, 1, 1, 4, 0, *outs, 0, 0, s) == 1       # null q
    assert lib.canopy_tree_verify(*args, 1, 1, 1, 4, 0, *outs, 0, 0, s) == 0
    torch.cuda.synchronize()
