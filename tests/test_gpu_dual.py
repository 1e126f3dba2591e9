"""Parity of the blocked solve sized for two workgroups per CU (waves=16; AUTO's kernel for trees
of 65-256 nodes with more than 256 (sequence, head) pairs) against the oracle: tree sizes across
the 16-node sub-block and 64-node block edges, tree shapes from a star to a 255-deep chain,
grouped heads with ragged batches (a sequence of one block, one of one node), malformed trees
and node counts, agreement with the one-per-CU blocked kernel, AUTO's dispatch to it, the
decode step through it, repeat determinism and the option checks."""
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


def _verify(canopy, d, solver="auto", waves=16, tree_len=None):
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


SIZES = [65, 79, 100, 127, 128, 129, 144, 191, 192, 193, 208, 255, 256]


@pytest.mark.parametrize("T", SIZES)
def test_sizes_random(canopy, T):
    inp = synth.make_inputs(2, 4, T, tree="random", dtype="bf16", seed=1200 + T)
    d = to_device(inp)
    ref = run_oracle(inp)
    _say("dual random", T)
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    assert_ell(ell, ref["ell"])
    _structure(inp, mask, depth, st)


@pytest.mark.parametrize("kind,kw,T", [("star", {}, 256), ("level", {"width": 64}, 256),
                                       ("level", {"width": 3}, 200), ("chain", {}, 256),
                                       ("skewed", {}, 256), ("random", {}, 150)])
def test_shapes(canopy, kind, kw, T):
    """A star (depth 1), level trees, the 255-deep chain (every diagonal sub-block at depth 15),
    the skewed tree."""
    inp = synth.make_inputs(2, 4, T, tree=kind, tree_kw=kw, dtype="bf16", seed=1300)
    d = to_device(inp)
    ref = run_oracle(inp)
    _say("dual shape", kind, kw, T)
    O, U, ell, mask, depth, st = _verify(canopy, d)
    assert_close_heads("O", O, ref["O"], TOL["bf16"])
    assert_close_heads("U", U, ref["U"], TOL["bf16"])
    _structure(inp, mask, depth, st)


def test_grouped_heads_and_ragged(canopy):
    """2 q/k heads for 8 value heads; sequences of T, 117, 64 (one block) and 1 nodes; outputs
    prefilled with a sentinel that rows past each sequence keep."""
    import torch
    B, HV, HK, T = 4, 8, 2, 230
    lens = np.array([T, 117, 64, 1], np.int32)
    inp = synth.make_inputs(B, HV, T, tree="random", dtype="bf16", seed=1400, HK=HK, tree_len=lens)
    d = to_device(inp)
    tl = torch.from_numpy(lens).cuda()
    O = torch.full((B, T, HV, 128), 777.0, device="cuda")
    U = torch.full_like(O, 777.0)
    L = torch.full((B, T, HV), 777.0, device="cuda")
    _say("dual grouped ragged")
    canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                       waves=16, out=(O, U, L), tree_len=tl)
    torch.cuda.synchronize()
    O, U = O.cpu().numpy(), U.cpu().numpy()
    ref = oracle.gdn_tree_ragged(inp["parent"], lens, inp["q"], inp["k"], inp["v"], inp["alpha"],
                                 inp["beta"], inp["S0"])
    for b in range(B):
        n = int(lens[b])
        assert_close_heads(f"O[b={b}]", O[b:b + 1, :n], ref["O"][b:b + 1, :n], TOL["bf16"])
        assert_close_heads(f"U[b={b}]", U[b:b + 1, :n], ref["U"][b:b + 1, :n], TOL["bf16"])
        assert (O[b, n:] == 777.0).all() and (U[b, n:] == 777.0).all()


def test_malformed_tree_and_length(canopy):
    """A parent that does not precede its child (status 1 + node) and a node count outside 1..T
    (status -1): NaN outputs for those sequences, the other within tolerance."""
    import torch
    inp = synth.make_inputs(3, 2, 150, tree="random", dtype="bf16", seed=1500)
    inp["parent"][1, 77] = 100
    d = to_device(inp)
    tl = torch.tensor([150, 150, 151], dtype=torch.int32, device="cuda")
    O, U, ell, mask, depth, st = _verify(canopy, d, tree_len=tl)
    assert st.tolist() == [0, 78, -1]
    for b in (1, 2):
        assert np.isnan(O[b]).all() and np.isnan(U[b]).all() and np.isnan(ell[b]).all()
    ok = dict(inp)
    for n in ("q", "k", "v", "alpha", "beta", "S0", "parent", "path", "path_len"):
        ok[n] = inp[n][:1]
    ok["B"] = 1
    ref = run_oracle(ok)
    assert_close_heads("O", O[:1], ref["O"], TOL["bf16"])
    assert_close_heads("U", U[:1], ref["U"], TOL["bf16"])


@pytest.mark.parametrize("T", [100, 256])
def test_agrees_with_one_per_cu_kernel(canopy, T):
    """The same forward substitution in the one-workgroup-per-CU blocked kernel (FWDSUB, 8
    waves): both in fp32 arithmetic from the same bf16 inputs, they agree to well inside the
    bf16 tolerance."""
    inp = synth.make_inputs(3, 8, T, tree="random", dtype="bf16", seed=1600 + T)
    d = to_device(inp)
    O_b, U_b = _verify(canopy, d, solver="fwdsub", waves=8)[:2]
    O_d, U_d = _verify(canopy, d, solver="fwdsub", waves=16)[:2]
    assert_close_heads("O", O_d, O_b, TOL["bf16"] / 20)
    assert_close_heads("U", U_d, U_b, TOL["bf16"] / 20)


def test_auto_dispatch_large_batch(canopy):
    """AUTO at B*H = 288 > 256 pairs runs this kernel: same bits as waves=16."""
    inp = synth.make_inputs(9, 32, 130, tree="random", dtype="bf16", seed=1700)
    d = to_device(inp)
    ref = run_oracle(inp)
    a = _verify(canopy, d, waves=0)
    w = _verify(canopy, d, waves=16)
    for x, y in zip(a, w):
        assert np.array_equal(x, y, equal_nan=True)
    assert_close_heads("O", a[0], ref["O"], TOL["bf16"])
    assert_close_heads("U", a[1], ref["U"], TOL["bf16"])


def test_repeat_bitwise(canopy):
    inp = synth.make_inputs(2, 4, 256, tree="random", dtype="bf16", seed=1800)
    d = to_device(inp)
    a = _verify(canopy, d)
    b = _verify(canopy, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_decode_step_through_it(canopy):
    """commit_verify with waves=16 after a 200-node tree: the commit kernel, then this verify
    on the committed state, against the oracle's path recurrence and per-path verify."""
    import torch
    prev = synth.make_inputs(2, 4, 200, tree="random", dtype="bf16", seed=1900)
    new = synth.make_inputs(2, 4, 180, tree="random", dtype="bf16", seed=1901)
    new["S0"] = prev["S0"]
    dp, dn = to_device(prev), to_device(new)
    _, U_prev, _ = canopy.tree_verify(dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], dp["S0"],
                                      dp["parent"], waves=16)
    Sn, pst, O, U, ell = canopy.commit_verify(dp["S0"], dp["k"], U_prev, dp["alpha"], dp["parent"],
                                              dp["path"], dp["path_len"], dn["q"], dn["k"], dn["v"],
                                              dn["alpha"], dn["beta"], dn["parent"], waves=16)
    torch.cuda.synchronize()
    S_ref, pst_ref = oracle_commit(prev)
    assert pst.cpu().numpy().tolist() == pst_ref.tolist()
    assert_close_state("S_new", Sn.cpu().numpy(), S_ref, TOL["bf16"])
    ref = oracle.gdn_tree(new["parent"], new["q"], new["k"], new["v"], new["alpha"], new["beta"], S_ref)
    assert_close_heads("O", O.cpu().numpy(), ref["O"], TOL["bf16"])
    assert_close_heads("U", U.cpu().numpy(), ref["U"], TOL["bf16"])


def test_options(canopy):
    """waves=16 takes bf16 inputs, T > 64 and the AUTO or FWDSUB solver only."""
    import torch
    cases = [("fp32", 100, "auto"), ("bf16", 64, "auto"), ("bf16", 100, "level"),
             ("bf16", 100, "neumann"), ("bf16", 100, "levelsync")]
    for dtype, T, solver in cases:
        inp = synth.make_inputs(1, 2, T, tree="random", dtype=dtype, seed=1950)
        d = to_device(inp)
        with pytest.raises(canopy.CanopyError):
            canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                               solver=solver, waves=16)
    torch.cuda.synchronize()
