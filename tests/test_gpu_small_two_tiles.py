"""Trees of at most 16 nodes at two 16-column tiles per wave (waves=16, and AUTO's choice for the
one-launch decode step past 384 (sequence, head) pairs with bf16 inputs).

Each wave runs the same per-tile arithmetic as at one tile per wave, in the same order, so the
outputs must equal the single-tile kernel's bit for bit; they are also held to the oracle at the
usual tolerances (max per-(batch, head) relative error 2e-3 for bf16 q/k/v, 1e-5 for fp32;
mask, depth and statuses bit-exact). Covered: verify alone and the one-launch step, bf16 and
fp32, the 1+3+12 top-k and 7-node binary trees, a 16-node chain (15 series terms), a single
node, grouped heads with ragged batches, a malformed tree, paths of every length class after
previous trees of up to 64 nodes, rejected paths, and the B=16 H=32 shape where AUTO picks
this width."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import TOL, assert_close_heads, assert_ell, run_oracle, to_device
from test_gpu_commit_verify import _check, _pair, _run

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


def _verify(canopy, d, waves, tree_len=None, solver="auto"):
    import torch
    tl = None if tree_len is None else torch.tensor(tree_len, dtype=torch.int32, device="cuda")
    B, T, HV = d["v"].shape[:3]
    O = torch.full((B, T, HV, 128), float("nan"), device="cuda")
    U = torch.full_like(O, float("nan"))
    ell = torch.full((B, T, HV), float("nan"), device="cuda")
    out = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                             solver=solver, waves=waves, structure=True, out=(O, U, ell),
                             tree_len=tl)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


CASES = [
    # (B, H, HK, T, tree, dtype, lens)
    (2, 8, None, 16, "topk", "bf16", None),
    (1, 2, None, 7, "binary7", "fp32", None),
    (2, 4, None, 16, "chain", "bf16", None),
    (3, 4, None, 1, "chain", "bf16", None),
    (3, 8, 2, 16, "random", "bf16", [16, 5, 1]),
    (3, 4, 2, 13, "random", "fp32", [13, 1, 7]),
]


@pytest.mark.parametrize("B,H,HK,T,tree,dtype,lens", CASES)
def test_verify_two_tiles(canopy, B, H, HK, T, tree, dtype, lens):
    kw = {"branching": (3, 4)} if tree == "topk" else None
    inp = synth.make_inputs(B, H, T, tree=tree, tree_kw=kw, dtype=dtype, seed=7100 + B * T + H,
                            HK=HK, tree_len=lens)
    d = to_device(inp)
    _say("verify two tiles", B, H, HK, T, tree, dtype, lens)
    for solver in ("auto", "neumann"):
        one = _verify(canopy, d, 1, lens, solver)
        two = _verify(canopy, d, 16, lens, solver)
        for name, x, y in zip(("O", "U", "ell", "status"), two[:3] + two[5:], one[:3] + one[5:]):
            assert np.array_equal(x, y, equal_nan=True), f"{solver} {name}: two tiles differ from one"
        for name, x, y in zip(("mask", "depth"), two[3:5], one[3:5]):  # rows inside each sequence
            for s, m in enumerate([T] * B if lens is None else lens):
                assert np.array_equal(x[s, :m], y[s, :m]), f"{solver} {name}: two tiles differ from one"
    O, U, ell = two[:3]
    if lens is None:
        ref = run_oracle(inp)
        assert_close_heads("O", O, ref["O"], TOL[dtype])
        assert_close_heads("U", U, ref["U"], TOL[dtype])
        assert_ell(ell, ref["ell"])
    else:
        import oracle
        ref = oracle.gdn_tree_ragged(inp["parent"], lens, inp["q"], inp["k"], inp["v"], inp["alpha"],
                                     inp["beta"], inp["S0"])
        pad = np.isnan(ref["O"])
        assert np.isnan(O[pad]).all() and np.isnan(U[pad]).all(), "a padding row was written"
        assert_close_heads("O", np.where(pad, 0.0, O), np.where(pad, 0.0, ref["O"]), TOL[dtype])
        assert_close_heads("U", np.where(pad, 0.0, U), np.where(pad, 0.0, ref["U"]), TOL[dtype])


def test_verify_two_tiles_malformed_tree(canopy):
    """A forward parent in sequence 1: its status and NaN outputs, the others untouched."""
    inp = synth.make_inputs(3, 4, 16, tree="random", dtype="bf16", seed=7200)
    inp["parent"][1, 7] = 9
    d = to_device(inp)
    _say("verify two tiles, malformed tree")
    O, U, ell, mask, depth, st = _verify(canopy, d, 16)
    assert st.tolist() == [0, 8, 0]
    assert np.isnan(O[1]).all() and np.isnan(U[1]).all() and np.isnan(ell[1]).all()
    assert (mask[1] == 0).all() and (depth[1] == 0).all()
    ref = run_oracle(synth.make_inputs(3, 4, 16, tree="random", dtype="bf16", seed=7200))
    assert_close_heads("O", O[[0, 2]], ref["O"][[0, 2]], TOL["bf16"])
    assert_close_heads("U", U[[0, 2]], ref["U"][[0, 2]], TOL["bf16"])


def _same(a, b, lens=None):
    """Bit-equal outputs; mask and depth only inside each sequence (rows past a ragged length
    are left unwritten)."""
    for name in ("S", "pst", "O", "U", "ell", "tst"):
        assert np.array_equal(a[name], b[name], equal_nan=True), f"{name}: two tiles differ from one"
    for name in ("mask", "depth"):
        n = [a[name].shape[1]] * a[name].shape[0] if lens is None else lens
        for s, m in enumerate(n):
            assert np.array_equal(a[name][s, :m], b[name][s, :m]), f"{name}: two tiles differ from one"


@pytest.mark.parametrize("Tp,plen,dtype", [(64, 0, "bf16"), (64, 1, "bf16"), (64, 5, "bf16"),
                                           (64, 16, "bf16"), (64, 64, "bf16"), (16, 16, "bf16"),
                                           (13, 6, "fp32")])
def test_step_two_tiles_path_lengths(canopy, Tp, plen, dtype):
    """The one-launch step after a chain, paths of every length class, at two tiles per wave:
    the single-tile kernel's bits and the oracle's values."""
    prev, new = _pair(2, 4, Tp, 16, dtype, 7300 + Tp + plen, tree_prev="chain")
    prev["path"][:] = -1
    prev["path"][:, :plen] = np.arange(plen)
    prev["path_len"][:] = plen
    _say("step two tiles, path length", Tp, plen, dtype)
    two = _run(canopy, prev, new, waves=16)
    one = _run(canopy, prev, new, waves=1)
    _same(two, one)
    _check(two, prev, new, dtype)


def test_step_two_tiles_grouped_ragged_rejected(canopy):
    """Grouped heads, ragged batches on both trees, a path that leaves the tree (sequence 1) and
    a bad previous length (sequence 2)."""
    lens_prev, lens = [40, 20, 0], [16, 9, 1]
    prev, new = _pair(3, 4, 40, 16, "bf16", 7400, HK=2, lens_prev=[40, 20, 1], lens=lens)
    prev["path"][1, 1] = prev["path"][1, 0]
    prev["path_len"][1] = max(prev["path_len"][1], 2)
    _say("step two tiles, grouped ragged rejected")
    two = _run(canopy, prev, new, lens_prev=lens_prev, lens=lens, waves=16)
    one = _run(canopy, prev, new, lens_prev=lens_prev, lens=lens, waves=1)
    _same(two, one, lens)
    assert two["pst"][0] == 0 and two["pst"][1] == 2 and two["pst"][2] == -1
    _check(two, prev, new, "bf16", lens_prev, lens)


def test_step_auto_b16(canopy):
    """B=16 H=32, the 1+3+12 top-k tree after another one: AUTO takes two tiles per wave for
    the one-launch step (4096 single-tile waves would not fit one pass at 3 per SIMD); same
    bits as waves=16 and waves=1, and the oracle over every (sequence, head)."""
    prev, new = _pair(16, 32, 16, 16, "bf16", 7500, tree_prev="topk", tree="topk")
    _say("step B=16 H=32 T=16 auto")
    auto = _run(canopy, prev, new)
    _same(auto, _run(canopy, prev, new, waves=16))
    _same(auto, _run(canopy, prev, new, waves=1))
    _check(auto, prev, new, "bf16")
