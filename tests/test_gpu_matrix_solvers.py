"""Parity of the matrix-form solvers (whole-tree Neumann series, squaring form, split design with
the inverse built once per (sequence, head)) through canopy_tree_verify_ws against the oracle:
the configurations, tile edges in both dtypes, a 256-node chain (depth 255), grouped heads and
ragged batches, malformed trees, and the workspace checks."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL, assert_close_heads, assert_close_state, assert_ell, oracle_commit,
                      run_oracle, to_device)

pytestmark = pytest.mark.gpu

SOLVERS = ("series", "squaring", "split")


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


def _say(*a):
    print("[gpu]", *a, flush=True)


def _verify(canopy, d, solver, tree_len=None):
    import torch
    out = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                             solver=solver, structure=True, tree_len=tree_len)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _structure(inp, mask, depth, st):
    dep_ref, mask_ref, st_ref = oracle.tree_structure(inp["parent"])
    assert np.array_equal(st, st_ref)
    assert np.array_equal(depth, dep_ref)
    assert np.array_equal(mask.view(np.uint32), mask_ref)


@pytest.mark.parametrize("solver", SOLVERS)
def test_binary7_fp32_and_commit(canopy, solver):
    """The 7-node binary tree in fp32, and the commit of path 0 -> 1 -> 3 from this solver's U
    equal to the oracle's state at node 3."""
    import torch
    inp = synth.make_inputs(1, 2, 7, tree="binary7", dtype="fp32", seed=0)
    inp["path"][:] = -1
    inp["path"][0, :3] = [0, 1, 3]
    inp["path_len"][:] = 3
    d = to_device(inp)
    ref = run_oracle(inp, accept=[3])
    _say("matrix binary7 fp32", solver)
    O, U, ell, mask, depth, st = _verify(canopy, d, solver)
    assert_close_heads("O", O, ref["O"], TOL["fp32"])
    assert_close_heads("U", U, ref["U"], TOL["fp32"])
    assert_ell(ell, ref["ell"])
    _structure(inp, mask, depth, st)
    Sn, pst = canopy.commit(d["S0"], d["k"], torch.from_numpy(U).cuda(), d["alpha"], d["parent"],
                            d["path"], d["path_len"])
    torch.cuda.synchronize()
    assert pst.cpu().numpy().tolist() == [0]
    assert_close_state("S_new", Sn.cpu().numpy(), ref["S_accept"], TOL["fp32"])


@pytest.mark.parametrize("solver", SOLVERS)
def test_topk16_bf16(canopy, solver):
    inp = synth.make_inputs(1, 32, 16, tree="topk", tree_kw={"branching": (3, 4)}, dtype="bf16", seed=1)
    d = to_device(inp)
    ref = run_oracle(inp)
    _say("matrix topk16", solver)
    O, U, ell, mask, depth, st = _verify(canopy, d, solver)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    _structure(inp, mask, depth, st)


EDGE_T = [1, 2, 15, 16, 17, 33, 64, 65, 100, 128, 129, 200, 255, 256]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T", EDGE_T)
def test_tile_edges(canopy, T, dtype):
    kinds = ["random", "skewed", "chain", "star", "level"]
    kind = kinds[T % len(kinds)]
    kw = {"width": 3} if kind == "level" else {}
    inp = synth.make_inputs(2, 2, T, tree=kind, tree_kw=kw, dtype=dtype, seed=700 + T)
    d = to_device(inp)
    ref = run_oracle(inp)
    for solver in SOLVERS:
        _say("matrix edge", T, dtype, kind, solver)
        O, U, ell, mask, depth, st = _verify(canopy, d, solver)
        assert_close_heads("O", O, ref["O"], TOL[dtype])
        assert_close_heads("U", U, ref["U"], TOL[dtype])
        assert_ell(ell, ref["ell"])
        _structure(inp, mask, depth, st)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_deep_chain(canopy, dtype):
    """A 256-node chain: depth 255, so 255 rounds of the series and 8 squaring factors."""
    inp = synth.make_inputs(1, 3, 256, tree="chain", dtype=dtype, seed=750)
    d = to_device(inp)
    ref = run_oracle(inp)
    for solver in SOLVERS:
        _say("matrix chain 256", dtype, solver)
        O, U, ell, mask, depth, st = _verify(canopy, d, solver)
        assert_close_heads("O", O, ref["O"], TOL[dtype])
        assert_close_heads("U", U, ref["U"], TOL[dtype])


@pytest.mark.parametrize("B,T,tree", [(4, 64, "skewed"), (2, 256, "random")])
def test_full_batches(canopy, B, T, tree):
    """Batches at the configurations' head count, every (b, h) pair against the oracle."""
    inp = synth.make_inputs(B, 32, T, tree=tree, dtype="bf16", seed=760 + B)
    d = to_device(inp)
    ref = run_oracle(inp)
    for solver in SOLVERS:
        _say("matrix batch", B, T, tree, solver)
        O, U, ell, mask, depth, st = _verify(canopy, d, solver)
        assert_close_heads("O", O, ref["O"], TOL["bf16"])
        assert_close_heads("U", U, ref["U"], TOL["bf16"])
        assert_ell(ell, ref["ell"])


@pytest.mark.parametrize("solver", SOLVERS)
def test_grouped_heads_and_ragged(canopy, solver):
    """2 q/k heads for 8 value heads; sequences of T, about T/2 and 1 nodes with NaN padding;
    outputs prefilled with a sentinel that padding rows keep."""
    import torch
    B, HV, HK, T = 3, 8, 2, 150
    lens = np.array([T, 77, 1], np.int32)
    inp = synth.make_inputs(B, HV, T, tree="random", dtype="bf16", seed=770, HK=HK, tree_len=lens)
    d = to_device(inp)
    tl = torch.from_numpy(lens).cuda()
    O = torch.full((B, T, HV, 128), 777.0, device="cuda")
    U = torch.full_like(O, 777.0)
    L = torch.full((B, T, HV), 777.0, device="cuda")
    _say("matrix grouped ragged", solver)
    canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                       solver=solver, out=(O, U, L), tree_len=tl)
    torch.cuda.synchronize()
    O, U = O.cpu().numpy(), U.cpu().numpy()
    ref = oracle.gdn_tree_ragged(inp["parent"], lens, inp["q"], inp["k"], inp["v"], inp["alpha"],
                                 inp["beta"], inp["S0"])
    for b in range(B):
        n = int(lens[b])
        assert_close_heads(f"O[b={b}]", O[b:b + 1, :n], ref["O"][b:b + 1, :n], TOL["bf16"])
        assert_close_heads(f"U[b={b}]", U[b:b + 1, :n], ref["U"][b:b + 1, :n], TOL["bf16"])
        assert (O[b, n:] == 777.0).all() and (U[b, n:] == 777.0).all()


@pytest.mark.parametrize("solver", SOLVERS)
def test_malformed_tree(canopy, solver):
    """A parent that does not precede its child: status 1 + node, NaN outputs for that
    sequence, the other sequence exact."""
    inp = synth.make_inputs(2, 2, 40, tree="random", dtype="bf16", seed=780)
    inp["parent"][1, 17] = 30
    d = to_device(inp)
    O, U, ell, mask, depth, st = _verify(canopy, d, solver)
    assert st.tolist() == [0, 18]
    assert np.isnan(O[1]).all() and np.isnan(U[1]).all()
    ok = dict(inp)
    for n in ("q", "k", "v", "alpha", "beta", "S0", "parent", "path", "path_len"):
        ok[n] = inp[n][:1]
    ok["B"] = 1
    ref = run_oracle(ok)
    assert_close_heads("O", O[:1], ref["O"], TOL["bf16"])


def test_workspace_checks(canopy):
    """The workspace entry point refuses a missing, misaligned or short workspace before any
    launch, and the fused solvers need none."""
    import torch
    lib = canopy.load()
    B, H, T = 1, 2, 100
    need = canopy.workspace_bytes(B, H, T, "split")
    assert need > 0 and canopy.workspace_bytes(B, H, T, "auto") == 0
    inp = synth.make_inputs(B, H, T, tree="random", dtype="bf16", seed=790)
    d = to_device(inp)
    O = torch.empty((B, T, H, 128), device="cuda")
    U = torch.empty_like(O)
    L = torch.empty((B, T, H), device="cuda")
    ws = torch.empty((need + 64,), dtype=torch.uint8, device="cuda")
    P = ctypes.c_void_p

    def call(wsp, nbytes, solver=6):
        return lib.canopy_tree_verify_ws(P(d["q"].data_ptr()), P(d["k"].data_ptr()), P(d["v"].data_ptr()),
                                         P(d["alpha"].data_ptr()), P(d["beta"].data_ptr()),
                                         P(d["S0"].data_ptr()), P(d["parent"].data_ptr()), None, B, H, H,
                                         T, 1, P(O.data_ptr()), P(U.data_ptr()), P(L.data_ptr()), None,
                                         None, None, solver, 0, wsp, nbytes, None)
    assert call(None, need) == 3
    assert call(P(ws.data_ptr()), need - 1) == 3
    assert call(P(ws.data_ptr() + 4), need) == 3
    assert call(None, 0, solver=0) == 0  # AUTO needs no workspace
    assert call(P(ws.data_ptr()), need) == 0
    torch.cuda.synchronize()
    ref = run_oracle(inp)
    assert_close_heads("O", O.cpu().numpy(), ref["O"], TOL["bf16"])


def test_errors_by_depth(canopy):
    """Every solve strategy across tree depths 1-255 (level trees of 256 nodes, widths 255 down
    to 1), bf16, B = 1, H = 32: the largest per-head relative error of O and U against the oracle
    stays within the bf16 tolerance; the errors are printed per depth and solver."""
    from _common import per_head_rel_err
    for W in (255, 128, 64, 32, 16, 8, 4, 2, 1):
        par = synth.level_tree(256, W)
        depth = int(synth.tree_depths(par).max())
        inp = synth.make_inputs(1, 32, 256, dtype="bf16", seed=11, parents=par)
        d = to_device(inp)
        ref = run_oracle(inp)
        errs = {}
        for solver in ("auto", "neumann") + SOLVERS:
            O, U, ell, mask, depth_o, st = _verify(canopy, d, solver)
            eo, eu = per_head_rel_err(O, ref["O"]), per_head_rel_err(U, ref["U"])
            errs[solver] = (eo, eu)
            assert eo <= TOL["bf16"] and eu <= TOL["bf16"], (depth, solver, eo, eu)
        _say("error by depth", depth, " ".join(f"{k}:O={v[0]:.2e},U={v[1]:.2e}" for k, v in errs.items()))
