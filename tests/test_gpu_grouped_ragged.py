"""Grouped value heads (q and k with fewer heads than v, the gates and the state) and ragged
batches (a node count per sequence, padding rows past it), through every verify kernel, the
commit and the serial baseline, against the oracle run on each sequence's own nodes with q and k
expanded to the value heads. Padding rows hold NaN, so any read of them would show."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close_heads, assert_close_state, assert_ell, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 777.0


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


def _say(*a):
    print("[gpu]", *a, flush=True)


def _upload(inp):
    import torch
    d = to_device(inp)
    if inp.get("tree_len") is not None:
        d["tree_len"] = torch.from_numpy(inp["tree_len"].astype(np.int32)).cuda()
    else:
        d["tree_len"] = None
    return d


def _verify(canopy, d, HV, solver="auto", waves=0):
    """Run verify into outputs prefilled with a sentinel; return numpy O, U, ell."""
    import torch
    B, T = d["parent"].shape
    O = torch.full((B, T, HV, 128), SENTINEL, device="cuda")
    U = torch.full_like(O, SENTINEL)
    L = torch.full((B, T, HV), SENTINEL, device="cuda")
    canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                       solver=solver, waves=waves, out=(O, U, L), tree_len=d["tree_len"])
    torch.cuda.synchronize()
    return O.cpu().numpy(), U.cpu().numpy(), L.cpu().numpy()


def _check_rows(inp, O, U, L, ref, tol):
    """Valid rows against the oracle, padding rows untouched."""
    B, T = inp["parent"].shape
    lens = inp["tree_len"] if inp["tree_len"] is not None else np.full(B, T)
    for b in range(B):
        n = int(lens[b])
        assert_close_heads(f"O[b={b}]", O[b:b + 1, :n], ref["O"][b:b + 1, :n], tol)
        assert_close_heads(f"U[b={b}]", U[b:b + 1, :n], ref["U"][b:b + 1, :n], tol)
        assert_ell(L[b, :n], ref["ell"][b, :n])
        assert (O[b, n:] == SENTINEL).all() and (U[b, n:] == SENTINEL).all(), f"padding written, b={b}"
        assert (L[b, n:] == SENTINEL).all(), f"padding ell written, b={b}"


# (T, dtype, solver, waves): one case per kernel tier
CASES = [
    (16, "bf16", "auto", 0),      # single-wave register kernel
    (7, "fp32", "neumann", 0),    # the same, fp32 inputs
    (40, "bf16", "auto", 0),      # wave-per-sub-block kernel, 17-64 nodes
    (64, "fp32", "fwdsub", 2),    # the same, fp32, two column tiles
    (130, "bf16", "auto", 0),     # wave-per-sub-block kernel, 65-256 nodes
    (200, "bf16", "fwdsub", 8),   # blocked kernel
    (100, "fp32", "auto", 0),     # blocked kernel, fp32
    (90, "bf16", "level", 0),     # blocked kernel, level solve
    (12, "bf16", "fwdsub", 0),    # blocked kernel for a small tree
]


@pytest.mark.parametrize("T,dtype,solver,waves", CASES)
def test_grouped_heads(canopy, T, dtype, solver, waves):
    """Two q/k heads serving eight value heads."""
    inp = synth.make_inputs(2, 8, T, tree="random", dtype=dtype, seed=1000 + T, HK=2)
    d = _upload(inp)
    _say("grouped", T, dtype, solver, waves)
    O, U, L = _verify(canopy, d, 8, solver, waves)
    ref = oracle.gdn_tree_ragged(inp["parent"], None, inp["q"], inp["k"], inp["v"], inp["alpha"],
                                 inp["beta"], inp["S0"])
    _check_rows(inp, O, U, L, ref, TOL[dtype])


@pytest.mark.parametrize("T,dtype,solver,waves", CASES)
def test_ragged_batch(canopy, T, dtype, solver, waves):
    """Three sequences of T, about half of T and 1 node, padding rows full of NaN, with grouped
    heads (HK = 2, HV = 4)."""
    lens = [T, max(1, T // 2 + 3), 1]
    inp = synth.make_inputs(3, 4, T, tree="skewed", dtype=dtype, seed=2000 + T, HK=2,
                            tree_len=lens)
    d = _upload(inp)
    _say("ragged", T, dtype, solver, waves, lens)
    O, U, L = _verify(canopy, d, 4, solver, waves)
    ref = oracle.gdn_tree_ragged(inp["parent"], inp["tree_len"], inp["q"], inp["k"], inp["v"],
                                 inp["alpha"], inp["beta"], inp["S0"])
    assert (ref["status"] == 0).all()
    _check_rows(inp, O, U, L, ref, TOL[dtype])


@pytest.mark.parametrize("T,solver,waves", [(16, "auto", 0), (40, "auto", 0), (130, "auto", 0),
                                            (130, "fwdsub", 8)])
def test_ragged_structure_and_bad_lengths(canopy, T, solver, waves):
    """Mask, depth and status of a ragged batch against brute force on each sequence's own
    nodes; lengths 0 and T + 1 give status -1 and NaN outputs over all T rows, without
    disturbing the valid sequence beside them."""
    import torch
    lens = np.array([0, T + 1, T - 5], np.int32)
    inp = synth.make_inputs(3, 2, T, tree="random", dtype="bf16", seed=3000 + T,
                            tree_len=[T, T, T - 5])
    inp["tree_len"] = lens
    d = _upload(inp)
    _say("bad lengths", T, solver, waves)
    O, U, L, mask, depth, st = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                  d["S0"], d["parent"], solver=solver,
                                                  waves=waves, structure=True,
                                                  tree_len=d["tree_len"])
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [-1, -1, 0]
    O, U, L = O.cpu().numpy(), U.cpu().numpy(), L.cpu().numpy()
    for b in (0, 1):
        assert np.isnan(O[b]).all() and np.isnan(U[b]).all() and np.isnan(L[b]).all()
    n = T - 5
    dep_ref, mask_ref, st_ref = oracle.tree_structure(inp["parent"][2:3, :n])
    assert st_ref[0] == 0
    W = (T + 31) // 32
    got_mask = mask.cpu().numpy().view(np.uint32)[2, :n]
    assert np.array_equal(depth.cpu().numpy()[2, :n], dep_ref[0])
    assert np.array_equal(got_mask[:, :mask_ref.shape[2]], mask_ref[0])
    assert not got_mask[:, mask_ref.shape[2]:W].any()
    ref = oracle.gdn_tree_ragged(inp["parent"], np.array([1, 1, n]), inp["q"], inp["k"], inp["v"],
                                 inp["alpha"], inp["beta"], inp["S0"])
    assert_close_heads("O", O[2:3, :n], ref["O"][2:3, :n], TOL["bf16"])
    assert_close_heads("U", U[2:3, :n], ref["U"][2:3, :n], TOL["bf16"])


@pytest.mark.parametrize("T,dtype", [(16, "bf16"), (100, "bf16"), (40, "fp32")])
def test_commit_grouped_ragged(canopy, T, dtype):
    """Commit with grouped heads on a ragged batch. Sequences: 0 and 1 random leaf paths (full
    and shorter tree); 2 a path whose second node lies past the sequence's length; 3 the whole
    chain; 4 a path longer than its sequence; 5 a length out of range. The statuses are the
    oracle's on each sequence's own nodes."""
    import torch
    n1 = T // 2 + 1
    lens = np.array([T, n1, n1, T, n1, T], np.int32)
    inp = synth.make_inputs(6, 4, T, tree="chain", dtype=dtype, seed=4000 + T, HK=2, tree_len=lens)
    inp["path"][2] = -1
    inp["path"][2, :2] = [0, n1]
    inp["path_len"][2] = 2
    inp["path"][3, :T] = np.arange(T)
    inp["path_len"][3] = T
    inp["path"][4, :n1 + 1] = np.arange(n1 + 1)
    inp["path_len"][4] = n1 + 1
    inp["tree_len"] = lens.copy()
    inp["tree_len"][5] = 0
    d = _upload(inp)
    _say("commit grouped ragged", T, dtype)
    _, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                                 tree_len=d["tree_len"])
    Sn, pst = canopy.commit(d["S0"], d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"],
                            tree_len=d["tree_len"])
    torch.cuda.synchronize()
    S_ref, st_ref = oracle.commit_ragged(inp["parent"], inp["tree_len"], inp["path"], inp["path_len"],
                                         inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    assert st_ref.tolist() == [0, 0, 2, 0, -1, -1]
    assert pst.cpu().numpy().tolist() == st_ref.tolist()
    Sn = Sn.cpu().numpy()
    ok = st_ref == 0
    assert np.isnan(Sn[~ok]).all()
    assert_close_state("S_new", Sn[ok], S_ref[ok], TOL[dtype])


@pytest.mark.parametrize("T", [9, 70])
def test_serial_grouped_ragged(canopy, T):
    """The serial baseline with grouped heads on a ragged batch, and its commit."""
    import torch
    lens = [T, T // 2, 1]
    inp = synth.make_inputs(3, 4, T, tree="random", dtype="bf16", seed=5000 + T, HK=1, tree_len=lens)
    d = _upload(inp)
    _say("serial grouped ragged", T)
    O, U, snap, st = canopy.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                          d["parent"], tree_len=d["tree_len"])
    Sn, pst = canopy.serial_commit(snap, d["S0"], d["parent"], d["path"], d["path_len"],
                                   tree_len=d["tree_len"])
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0, 0, 0]
    ref = oracle.gdn_tree_ragged(inp["parent"], inp["tree_len"], inp["q"], inp["k"], inp["v"],
                                 inp["alpha"], inp["beta"], inp["S0"])
    O, U = O.cpu().numpy(), U.cpu().numpy()
    for b, n in enumerate(lens):
        assert_close_heads("O", O[b:b + 1, :n], ref["O"][b:b + 1, :n], TOL["bf16"])
        assert_close_heads("U", U[b:b + 1, :n], ref["U"][b:b + 1, :n], TOL["bf16"])
    S_ref, st_ref = oracle.commit_ragged(inp["parent"], inp["tree_len"], inp["path"], inp["path_len"],
                                         inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    assert pst.cpu().numpy().tolist() == st_ref.tolist() == [0, 0, 0]
    assert_close_state("S_new", Sn.cpu().numpy(), S_ref, TOL["bf16"])


def test_tree_prep_ragged(canopy):
    """Standalone preprocessing of a ragged batch: ell, mask and depth of each sequence's own
    nodes; padding rows of ell are not written."""
    import torch
    T = 150
    lens = [150, 64, 65, 1]
    inp = synth.make_inputs(4, 3, T, tree="random", dtype="fp32", seed=6000, tree_len=lens)
    d = _upload(inp)
    mask, depth, ell, st = canopy.tree_prep(d["parent"], d["alpha"], tree_len=d["tree_len"])
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0, 0, 0, 0]
    ref = oracle.gdn_tree_ragged(inp["parent"], inp["tree_len"], inp["q"], inp["k"], inp["v"],
                                 inp["alpha"], inp["beta"], inp["S0"])
    mask = mask.cpu().numpy().view(np.uint32)
    depth, ell = depth.cpu().numpy(), ell.cpu().numpy()
    for b, n in enumerate(lens):
        dep_ref, mask_ref, _ = oracle.tree_structure(inp["parent"][b:b + 1, :n])
        assert np.array_equal(depth[b, :n], dep_ref[0])
        assert np.array_equal(mask[b, :n, :mask_ref.shape[2]], mask_ref[0])
        assert_ell(ell[b, :n], ref["ell"][b, :n])
