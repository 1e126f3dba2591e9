"""Parity of the chain-decomposed hybrid (heavy-light chains, each serial, chains of a level in
parallel) against the oracle's per-path recurrence, through the C ABI, at each workgroup width
(8 or 16 waves for one sequence's heads, 4 beyond)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL, assert_close_heads, assert_close_state, oracle_commit, run_oracle,
                      slice_inputs, to_device)

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


TREES = [
    (1, 2, 7, "binary7", "fp32", {}),
    (1, 4, 16, "topk", "bf16", {"branching": (3, 4)}),
    (2, 3, 64, "skewed", "bf16", {}),
    (2, 2, 100, "chain", "fp32", {}),
    (1, 3, 50, "star", "bf16", {}),
    (2, 2, 200, "random", "bf16", {}),
    (1, 2, 256, "level", "fp32", {"width": 4}),
    (2, 20, 40, "random", "bf16", {}),      # more than 32 (sequence, head) pairs: 4 waves
    (1, 32, 130, "skewed", "bf16", {}),     # one sequence, T > 64: 16 waves
]


@pytest.mark.parametrize("B,H,T,tree,dtype,kw", TREES)
def test_hybrid_matches_oracle(canopy, B, H, T, tree, dtype, kw):
    import torch
    inp = synth.make_inputs(B, H, T, tree=tree, dtype=dtype, seed=600 + T, tree_kw=kw)
    d = to_device(inp)
    _say("hybrid", B, H, T, tree, dtype)
    O, U, snap, st = canopy.hybrid_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                          d["parent"])
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0] * B
    ref = run_oracle(inp)
    assert_close_heads("O", O.cpu().numpy(), ref["O"], TOL[dtype])
    assert_close_heads("U", U.cpu().numpy(), ref["U"], TOL[dtype])
    # its U commits like the parallel path's
    Sn, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
    torch.cuda.synchronize()
    S_ref, st_ref = oracle_commit(inp)
    assert pst.cpu().numpy().tolist() == st_ref.tolist() == [0] * B
    assert_close_state("S_new", Sn.cpu().numpy(), S_ref, TOL[dtype])


def test_hybrid_fork_snapshots_and_forest(canopy):
    """Two roots, branching at several depths: every fork node's snapshot equals the oracle's
    state there, and both trees of the forest start from S0."""
    import torch
    par = np.array([-1, 0, 0, 1, 1, 3, -1, 6, 6, 7, 2, 2, 11, 11, 5, 14], np.int32)
    T = len(par)
    inp = synth.make_inputs(1, 2, T, dtype="fp32", seed=611, parents=par)
    d = to_device(inp)
    O, U, snap, st = canopy.hybrid_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                          d["parent"])
    torch.cuda.synchronize()
    ref = run_oracle(inp, all_states=True)
    assert_close_heads("O", O.cpu().numpy(), ref["O"], TOL["fp32"])
    assert_close_heads("U", U.cpu().numpy(), ref["U"], TOL["fp32"])
    nch = np.bincount(par[par >= 0], minlength=T)
    forks = np.nonzero(nch >= 2)[0]
    assert len(forks) >= 4
    snap = snap.cpu().numpy()
    for f in forks:
        assert_close_state(f"snapshot {f}", snap[:, f], ref["S_all"][:, f], TOL["fp32"])


def test_hybrid_grouped_ragged(canopy):
    import torch
    lens = [90, 33, 1]
    inp = synth.make_inputs(3, 4, 90, tree="random", dtype="bf16", seed=612, HK=2, tree_len=lens)
    d = to_device(inp)
    tl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    O, U, _, st = canopy.hybrid_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                       d["parent"], tree_len=tl)
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0, 0, 0]
    ref = oracle.gdn_tree_ragged(inp["parent"], inp["tree_len"], inp["q"], inp["k"], inp["v"],
                                 inp["alpha"], inp["beta"], inp["S0"])
    O, U = O.cpu().numpy(), U.cpu().numpy()
    for b, n in enumerate(lens):
        assert_close_heads("O", O[b:b + 1, :n], ref["O"][b:b + 1, :n], TOL["bf16"])
        assert_close_heads("U", U[b:b + 1, :n], ref["U"][b:b + 1, :n], TOL["bf16"])


def test_hybrid_malformed_tree(canopy):
    import torch
    inp = synth.make_inputs(2, 1, 12, tree="random", dtype="fp32", seed=613)
    inp["parent"][1, 7] = 9
    d = to_device(inp)
    O, U, _, st = canopy.hybrid_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                       d["parent"])
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0, 8]
    assert np.isnan(O[1].cpu().numpy()).all() and np.isnan(U[1].cpu().numpy()).all()
    ref = run_oracle(slice_inputs(inp, [0], [0]))
    assert_close_heads("O", O[:1].cpu().numpy(), ref["O"], TOL["fp32"])
