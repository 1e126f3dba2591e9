"""The fused decode step (commit of the previous tree's accepted path, then the verify of a new
tree from the committed state) through the C ABI, against the oracle's path recurrence followed
by its per-path verify, and against the two separate calls.

Tolerances as for the separate calls: max per-(batch, head) relative error 2e-3 for bf16 q/k/v
(1e-5 for fp32) for O, U and the committed state against the oracle; mask, depth and both
statuses bit-exact. Covered: the one-launch form (new trees of at most 16 nodes after previous
trees of at most 64) at the 1+3+12 top-k shape and for 17-64-node trees with narrow
workgroups, paths of 0, 1..4 and more than 4 positions, grouped heads and ragged batches, fp32
inputs, rejected paths, the state committed in place and one U buffer for both trees; and the
two-launch form for the other shapes."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close_heads, assert_close_state, to_device

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


def _np(t):
    return t.detach().cpu().numpy()


def _pair(B, H, Tp, T, dtype, seed, tree_prev="random", tree="random", HK=None, lens_prev=None,
          lens=None):
    """A previous tree (its path drawn by synth) and a new tree sharing the previous S0."""
    kwp = {"branching": (3, 4)} if tree_prev == "topk" else None
    kw = {"branching": (3, 4)} if tree == "topk" else None
    prev = synth.make_inputs(B, H, Tp, tree=tree_prev, tree_kw=kwp, dtype=dtype, seed=seed, HK=HK,
                             tree_len=lens_prev)
    new = synth.make_inputs(B, H, T, tree=tree, tree_kw=kw, dtype=dtype, seed=seed + 1, HK=HK,
                            tree_len=lens)
    new["S0"] = prev["S0"]
    return prev, new


def _run(canopy, prev, new, lens_prev=None, lens=None, S_in_place=False, share_U=False, **kw):
    import torch
    dp, dn = to_device(prev), to_device(new)
    tlp = None if lens_prev is None else torch.tensor(lens_prev, dtype=torch.int32, device="cuda")
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    _, U_prev, _ = canopy.tree_verify(dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], dp["S0"],
                                      dp["parent"], tree_len=tlp)
    B, T, HV = new["v"].shape[:3]
    O = torch.full((B, T, HV, 128), float("nan"), device="cuda")
    U = U_prev if share_U else torch.full_like(O, float("nan"))
    ell = torch.full((B, T, HV), float("nan"), device="cuda")
    S0 = dp["S0"].clone()
    Sn, pst, O, U, ell, mask, depth, tst = canopy.commit_verify(
        S0, dp["k"], U_prev, dp["alpha"], dp["parent"], dp["path"], dp["path_len"], dn["q"], dn["k"],
        dn["v"], dn["alpha"], dn["beta"], dn["parent"], structure=True, out=(O, U, ell),
        S_out=S0 if S_in_place else None, tree_len_prev=tlp, tree_len=tl, **kw)
    torch.cuda.synchronize()
    return dict(S=_np(Sn), pst=_np(pst), O=_np(O), U=_np(U), ell=_np(ell), mask=_np(mask),
                depth=_np(depth), tst=_np(tst), dev=(dp, dn, tlp, tl, U_prev))


def _separate(canopy, r, **kw):
    import torch
    dp, dn, tlp, tl, U_prev = r["dev"]
    Sn, pst = canopy.commit(dp["S0"], dp["k"], U_prev, dp["alpha"], dp["parent"], dp["path"],
                            dp["path_len"], tree_len=tlp)
    O, U, ell = canopy.tree_verify(dn["q"], dn["k"], dn["v"], dn["alpha"], dn["beta"], Sn, dn["parent"],
                                   tree_len=tl, **kw)
    torch.cuda.synchronize()
    return dict(S=_np(Sn), pst=_np(pst), O=_np(O), U=_np(U), ell=_np(ell))


def _oracle(prev, new, lens_prev=None, lens=None):
    S_ref, pst = oracle.commit_ragged(prev["parent"], lens_prev, prev["path"], prev["path_len"],
                                      prev["k"], prev["v"], prev["alpha"], prev["beta"], prev["S0"])
    ref = oracle.gdn_tree_ragged(new["parent"], lens, new["q"], new["k"], new["v"], new["alpha"],
                                 new["beta"], np.where(np.isnan(S_ref), 0.0, S_ref))
    return S_ref, pst, ref


def _check(r, prev, new, dtype, lens_prev=None, lens=None):
    tol = TOL[dtype]
    S_ref, pst_ref, ref = _oracle(prev, new, lens_prev, lens)
    assert r["pst"].tolist() == pst_ref.tolist()
    good = pst_ref == 0
    assert_close_state("S_new", r["S"][good], S_ref[good], tol)
    assert np.isnan(r["S"][~good]).all()
    pad = np.isnan(ref["O"])  # rows past a sequence's length stay unwritten
    for name in ("O", "U"):
        x = r[name]
        assert np.isnan(x[pad]).all(), f"{name}: a padding row was written"
        xg = np.where(pad, 0.0, x)[good]
        assert_close_heads(name, xg, np.where(pad, 0.0, ref[name])[good], tol)
        assert np.isnan(x[~good][~pad[~good]]).all(), f"{name}: rejected path, outputs not NaN"
    dep, mask, st = oracle.tree_structure(new["parent"]) if lens is None else (None, None, None)
    if lens is None:
        assert r["tst"].tolist() == st.tolist()
        assert np.array_equal(r["depth"], dep)
        assert np.array_equal(r["mask"].view(np.uint32), mask)


def test_topk16_step(canopy):
    """The 1+3+12 top-k tree after another one, B=1 H=32 bf16: the one-launch form, against the
    oracle and the two separate calls."""
    prev, new = _pair(1, 32, 16, 16, "bf16", 6000, tree_prev="topk", tree="topk")
    _say("topk16 step")
    r = _run(canopy, prev, new)
    _check(r, prev, new, "bf16")
    s = _separate(canopy, r)
    assert r["pst"].tolist() == s["pst"].tolist()
    for name in ("S", "O", "U"):
        err = np.max(np.abs(r[name] - s[name])) / max(1e-30, np.max(np.abs(s[name])))
        assert err < 1e-5, f"{name}: fused and separate differ by {err:.2e}"
    assert np.array_equal(r["ell"], s["ell"])


@pytest.mark.parametrize("Tp,plen", [(64, 0), (64, 1), (64, 3), (64, 4), (64, 5), (64, 9), (64, 16),
                                     (64, 40), (64, 64), (16, 0), (16, 1), (16, 5), (16, 16), (9, 9)])
def test_path_lengths(canopy, Tp, plen):
    """A chain before a random 16-node tree, paths of every length class: none, one operand
    group, a partial and a full group, up to every position. Previous trees of up to 64 nodes
    read the path's nodes after the path; those of up to 16 read every node up front."""
    B, H = 2, 4
    prev, new = _pair(B, H, Tp, 16, "bf16", 6100 + plen + Tp, tree_prev="chain")
    prev["path"][:] = -1
    prev["path"][:, :plen] = np.arange(plen)
    prev["path_len"][:] = plen
    _say("path length", plen)
    r = _run(canopy, prev, new)
    _check(r, prev, new, "bf16")
    if plen == 0:
        assert np.array_equal(r["S"], prev["S0"].astype(np.float32)), "an empty path must keep S0"


@pytest.mark.parametrize("dtype,Tp", [("bf16", 40), ("fp32", 40), ("bf16", 16), ("fp32", 13)])
def test_grouped_ragged(canopy, dtype, Tp):
    """Grouped heads (2 q/k heads, 4 value heads) and ragged batches on both trees (padding
    rows of the previous tree full of NaN, its U past each length unwritten)."""
    lens_prev, lens = [Tp, 9, 1], [16, 5, 1]
    prev, new = _pair(3, 4, Tp, 16, dtype, 6200 + Tp, HK=2, lens_prev=lens_prev, lens=lens)
    _say("grouped ragged", dtype, Tp)
    r = _run(canopy, prev, new, lens_prev=lens_prev, lens=lens)
    _check(r, prev, new, dtype, lens_prev, lens)


def test_binary7_fp32(canopy):
    """The 7-node binary tree twice, fp32, B=1 H=2."""
    prev, new = _pair(1, 2, 7, 7, "fp32", 6300, tree_prev="binary7", tree="binary7")
    prev["path"][:] = -1
    prev["path"][0, :3] = [0, 1, 3]
    prev["path_len"][:] = 3
    for solver in ("auto", "neumann"):
        for waves in (1, 8):
            _say("binary7 fp32", solver, waves)
            r = _run(canopy, prev, new, solver=solver, waves=waves)
            _check(r, prev, new, "fp32")


@pytest.mark.parametrize("Tp", [30, 12])
def test_rejected_paths(canopy, Tp):
    """A path that leaves the tree, a path_len past the tree and a bad tree_len: status as in
    the commit, NaN state and NaN outputs for those sequences only."""
    B, H = 4, 4
    lens_prev = [Tp, Tp, Tp, 0]
    prev, new = _pair(B, H, Tp, 12, "bf16", 6400 + Tp, lens_prev=[Tp, Tp, Tp, Tp])
    prev["path"][1, 1] = prev["path"][1, 0]  # position 1 is not a child of position 0
    prev["path_len"][1] = max(prev["path_len"][1], 2)
    prev["path_len"][2] = Tp + 1  # longer than the tree
    _say("rejected paths")
    r = _run(canopy, prev, new, lens_prev=lens_prev)
    S_ref, pst_ref, _ = _oracle(prev, new, lens_prev)
    assert r["pst"].tolist() == pst_ref.tolist()
    assert r["pst"][0] == 0 and r["pst"][1] == 2 and r["pst"][2] == -1 and r["pst"][3] == -1
    _check(r, prev, new, "bf16", lens_prev)


def test_in_place_and_shared_U(canopy):
    """S_new written over S0 and one U buffer for both trees (equal sizes) give the same bits
    as separate buffers."""
    prev, new = _pair(2, 8, 16, 16, "bf16", 6500)
    _say("in place, shared U")
    a = _run(canopy, prev, new)
    b = _run(canopy, prev, new, S_in_place=True, share_U=True)
    for name in ("S", "pst", "O", "U", "ell"):
        assert np.array_equal(a[name], b[name], equal_nan=True), name


@pytest.mark.parametrize("B,H,Tp,T", [(2, 4, 100, 16), (2, 4, 64, 130), (3, 16, 16, 40), (3, 48, 30, 64),
                                     (2, 4, 100, 40)])
def test_two_launch_form(canopy, B, H, Tp, T):
    """Shapes outside the one-launch forms (a previous tree past 64 nodes, a new tree past 64,
    17-64-node trees with wide workgroups): the commit kernel, then the verify kernel."""
    prev, new = _pair(B, H, Tp, T, "bf16", 6600 + Tp + T + H)
    _say("two launches", B, H, Tp, T)
    r = _run(canopy, prev, new)
    _check(r, prev, new, "bf16")


@pytest.mark.parametrize("T,Tp,plen,dtype", [(17, 16, 3, "bf16"), (40, 16, 16, "bf16"), (64, 64, 0, "bf16"),
                                             (64, 64, 7, "bf16"), (33, 64, 64, "bf16"), (48, 40, 13, "fp32"),
                                             (64, 12, 5, "fp32")])
def test_mid_one_launch(canopy, T, Tp, plen, dtype):
    """The one-launch form for new trees of 17 to 64 nodes (narrow workgroups, B * H <= 32):
    chains before random trees, paths of every length class."""
    B, H = 2, 4
    prev, new = _pair(B, H, Tp, T, dtype, 6700 + T + Tp + plen, tree_prev="chain")
    prev["path"][:] = -1
    prev["path"][:, :plen] = np.arange(plen)
    prev["path_len"][:] = plen
    _say("17-64 one launch", T, Tp, plen, dtype)
    r = _run(canopy, prev, new)
    _check(r, prev, new, dtype)
    if plen == 0:
        assert np.array_equal(r["S"], prev["S0"].astype(np.float32)), "an empty path must keep S0"
    s = _separate(canopy, r)
    for name in ("S", "O", "U"):
        err = np.max(np.abs(r[name] - s[name])) / max(1e-30, np.max(np.abs(s[name])))
        assert err < 1e-5, f"{name}: fused and separate differ by {err:.2e}"


@pytest.mark.parametrize("B,H,T,Tp", [(2, 48, 64, 30), (4, 32, 64, 64), (2, 64, 49, 20)])
def test_mid_one_launch_two_tiles(canopy, B, H, T, Tp):
    """The one-launch form at two column tiles per workgroup (65-128 heads, 49-64 nodes): against
    the oracle and the two separate calls."""
    prev, new = _pair(B, H, Tp, T, "bf16", 6750 + B * H + T)
    _say("17-64 one launch, two tiles", B, H, T, Tp)
    r = _run(canopy, prev, new)
    _check(r, prev, new, "bf16")
    s = _separate(canopy, r)
    for name in ("S", "O", "U"):
        err = np.max(np.abs(r[name] - s[name])) / max(1e-30, np.max(np.abs(s[name])))
        assert err < 1e-5, f"{name}: fused and separate differ by {err:.2e}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_mid_grouped_ragged_rejected(canopy, dtype):
    """The 17-64 one-launch form with grouped heads, ragged batches on both trees and a rejected
    path (sequence 1) and a bad length (sequence 2)."""
    lens_prev, lens = [50, 20, 0], [40, 17, 1]
    prev, new = _pair(3, 4, 50, 40, dtype, 6800, HK=2, lens_prev=[50, 20, 1], lens=lens)
    prev["path"][1, 1] = prev["path"][1, 0]
    prev["path_len"][1] = max(prev["path_len"][1], 2)
    _say("17-64 grouped ragged rejected", dtype)
    r = _run(canopy, prev, new, lens_prev=lens_prev, lens=lens)
    assert r["pst"][0] == 0 and r["pst"][1] == 2 and r["pst"][2] == -1
    _check(r, prev, new, dtype, lens_prev, lens)
