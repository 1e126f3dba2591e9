"""Parity of the level-synchronous gather solve (CANOPY_SOLVE_LEVELSYNC) against the oracle: tree
sizes across the 16-node batch edges and the 64-node block edges, tree shapes from a star to the
deepest tree that fits, grouped heads, ragged batches, malformed trees, trees that exceed the
tables (the blocked solve takes them), agreement with the blocked solve, the commit from its U,
and the B=16 H=32 T=256 random-tree layer over the full grid."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL, assert_close_heads, assert_close_state, assert_ell, oracle_commit,
                      run_oracle, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


def _say(*a):
    print("[gpu]", *a, flush=True)


def _verify(canopy, d, solver="levelsync", waves=0, tree_len=None):
    import torch
    out = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                             solver=solver, waves=waves, structure=True, tree_len=tree_len)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _structure(inp, mask, depth, st):
    dep_ref, mask_ref, st_ref = oracle.tree_structure(inp["parent"])
    assert np.array_equal(st, st_ref)
    assert np.array_equal(depth, dep_ref)
    assert np.array_equal(mask.view(np.uint32), mask_ref)


def _depth_stats(parent):
    """(sum of depths, nodes with a child) of one tree: the two quantities the tables bound."""
    T = len(parent)
    d = np.zeros(T, np.int64)
    for i in range(T):
        if parent[i] >= 0:
            d[i] = d[parent[i]] + 1
    return int(d.sum()), len({int(p) for p in parent if p >= 0})


SIZES = [1, 2, 15, 16, 17, 33, 64, 65, 100, 128, 129, 191, 192, 193, 255, 256]


@pytest.mark.parametrize("T", SIZES)
def test_sizes_random(canopy, T):
    inp = synth.make_inputs(2, 4, T, tree="random", dtype="bf16", seed=900 + T)
    d = to_device(inp)
    ref = run_oracle(inp)
    _say("levelsync random", T)
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    assert_ell(ell, ref["ell"])
    _structure(inp, mask, depth, st)


@pytest.mark.parametrize("kind,kw", [("star", {}), ("topk", {"branching": (3, 4)}),
                                     ("level", {"width": 64}), ("level", {"width": 40}),
                                     ("chain", {}), ("skewed", {})])
def test_shapes(canopy, kind, kw):
    """Shapes at T = 256 (top-k: its 16-node tree). The chain (depth 255, 32640 pairs) and the
    skewed tree exceed the pair table and run the blocked solve; the others fit."""
    T = 16 if kind == "topk" else 256
    inp = synth.make_inputs(2, 4, T, tree=kind, tree_kw=kw, dtype="bf16", seed=950)
    d = to_device(inp)
    ref = run_oracle(inp)
    for b in range(2):
        _say("levelsync shape", kind, kw, "tree", b, "(pairs, internal) =", _depth_stats(inp["parent"][b]))
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    _structure(inp, mask, depth, st)


def _levels_tree(last_parents):
    """Root; 64 nodes under it; 64 under those; 64 under those; 63 more under the first
    `last_parents` nodes of the third level: 1 + 64 + 64 + last_parents nodes with a child."""
    T = 256
    par = np.full(T, -1, np.int64)
    par[1:65] = 0
    par[65:129] = np.arange(1, 65)
    par[129:193] = np.arange(65, 129)
    par[193:] = 129 + (np.arange(193, T) - 193) % last_parents
    return par


def _broom_tree(deeper):
    """A chain 0..9 and 246 leaves under node 9 (depth 10), of which `deeper` hang under node 10
    instead (depth 11): 2505 + deeper (node, ancestor) pairs."""
    T = 256
    par = np.full(T, -1, np.int64)
    par[1:10] = np.arange(0, 9)
    par[10:] = 9
    par[T - deeper:] = 10
    return par


@pytest.mark.parametrize("par,pairs,internal", [
    (_levels_tree(31), 636, 160),
    (_levels_tree(32), 636, 161),
    (_broom_tree(55), 2560, 11),
    (_broom_tree(56), 2561, 11),
])
def test_table_limits(canopy, par, pairs, internal):
    """Trees at and just past each table bound (2560 pairs, 160 nodes with a child): the first
    and third fit, the others run the blocked solve; all match the oracle."""
    assert _depth_stats(par) == (pairs, internal)
    inp = synth.make_inputs(1, 2, len(par), dtype="bf16", seed=960, parents=par)
    d = to_device(inp)
    ref = run_oracle(inp)
    _say("levelsync table limits: pairs", pairs, "internal", internal)
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])


def test_grouped_heads_and_ragged(canopy):
    """2 q/k heads for 8 value heads; sequences of T, about T/2 and 1 nodes; outputs prefilled
    with a sentinel that rows past each sequence keep."""
    import torch
    B, HV, HK, T = 3, 8, 2, 230
    lens = np.array([T, 117, 1], np.int32)
    inp = synth.make_inputs(B, HV, T, tree="random", dtype="bf16", seed=970, HK=HK, tree_len=lens)
    d = to_device(inp)
    tl = torch.from_numpy(lens).cuda()
    O = torch.full((B, T, HV, 128), 777.0, device="cuda")
    U = torch.full_like(O, 777.0)
    L = torch.full((B, T, HV), 777.0, device="cuda")
    _say("levelsync grouped ragged")
    canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                       solver="levelsync", out=(O, U, L), tree_len=tl)
    torch.cuda.synchronize()
    O, U = O.cpu().numpy(), U.cpu().numpy()
    ref = oracle.gdn_tree_ragged(inp["parent"], lens, inp["q"], inp["k"], inp["v"], inp["alpha"],
                                 inp["beta"], inp["S0"])
    for b in range(B):
        n = int(lens[b])
        assert_close_heads(f"O[b={b}]", O[b:b + 1, :n], ref["O"][b:b + 1, :n], TOL["bf16"])
        assert_close_heads(f"U[b={b}]", U[b:b + 1, :n], ref["U"][b:b + 1, :n], TOL["bf16"])
        assert (O[b, n:] == 777.0).all() and (U[b, n:] == 777.0).all()


def test_malformed_tree(canopy):
    """A parent that does not precede its child: status 1 + node, NaN outputs for that sequence,
    the other sequence within tolerance."""
    inp = synth.make_inputs(2, 2, 150, tree="random", dtype="bf16", seed=980)
    inp["parent"][1, 77] = 100
    d = to_device(inp)
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert st.tolist() == [0, 78]
    assert np.isnan(O[1]).all() and np.isnan(U[1]).all()
    ok = dict(inp)
    for n in ("q", "k", "v", "alpha", "beta", "S0", "parent", "path", "path_len"):
        ok[n] = inp[n][:1]
    ok["B"] = 1
    ref = run_oracle(ok)
    assert_close_heads("O", O[:1], ref["O"], TOL["bf16"])


def test_agrees_with_blocked_solve(canopy):
    """With more than 128 (sequence, head) pairs AUTO runs the blocked solve (forward
    substitution over 16-node sub-blocks of 64-node blocks): the gather solve agrees with it to well inside the bf16 tolerance (both in fp32
    arithmetic from the same bf16 inputs)."""
    inp = synth.make_inputs(5, 32, 200, tree="random", dtype="bf16", seed=990)
    d = to_device(inp)
    O_a, U_a = _verify(canopy, d, solver="auto")[:2]
    O_l, U_l = _verify(canopy, d, solver="levelsync")[:2]
    assert_close_heads("O", O_l, O_a, TOL["bf16"] / 4)
    assert_close_heads("U", U_l, U_a, TOL["bf16"] / 4)


def test_options(canopy):
    """LEVELSYNC takes bf16 inputs and 0 or 8 waves only."""
    import torch
    lib = canopy.load()
    inp = synth.make_inputs(1, 2, 100, tree="random", dtype="fp32", seed=991)
    d = to_device(inp)
    with pytest.raises(canopy.CanopyError):
        canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                           solver="levelsync")
    inp = synth.make_inputs(1, 2, 100, tree="random", dtype="bf16", seed=991)
    d = to_device(inp)
    with pytest.raises(canopy.CanopyError):
        canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                           solver="levelsync", waves=4)
    torch.cuda.synchronize()
    del lib


def test_commit_from_levelsync_U(canopy):
    import torch
    inp = synth.make_inputs(2, 4, 256, tree="random", dtype="bf16", seed=995)
    d = to_device(inp)
    O, U, ell, mask, depth, st = _verify(canopy, d)
    Sn, pst = canopy.commit(d["S0"], d["k"], torch.from_numpy(U).cuda(), d["alpha"], d["parent"],
                            d["path"], d["path_len"])
    torch.cuda.synchronize()
    S_or, st_or = oracle_commit(inp)
    assert np.array_equal(pst.cpu().numpy(), st_or)
    assert_close_state("S_new", Sn.cpu().numpy(), S_or, TOL["bf16"])


def test_config_random256_b16_full_grid(canopy):
    """The benchmark's large-tree layer (B=16 H=32 T=256 random recursive trees, bf16) through
    the gather solve, every (b, h) pair."""
    import time
    inp = synth.make_inputs(16, 32, 256, tree="random", dtype="bf16", seed=3)
    fits = [_depth_stats(inp["parent"][b]) for b in range(16)]
    _say("random256 B16 (pairs, internal) per tree:", fits)
    d = to_device(inp)
    t0 = time.perf_counter()
    ref = run_oracle(inp)
    _say("random256 B16 oracle over the full grid: %.2f s" % (time.perf_counter() - t0))
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    assert_ell(ell, ref["ell"])
    _structure(inp, mask, depth, st)
