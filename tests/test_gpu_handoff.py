"""A lost hand-off between the waves of a workgroup is visible: with the wait bound set to 0 from
the host, every wave that waits for another wave's result gives up at once, writes NaN for the
rows it computes and sets tree status -2, while every kernel still ends normally. The rows that
need no hand-off keep their oracle values, and restoring the default bound restores parity."""
import numpy as np
import pytest

import synth
from gpu_util import TOL, assert_close_heads, run_oracle, to_device

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


def _with_bound_zero(canopy, fn):
    prev = canopy.set_wait_bound(0)
    try:
        out = fn()
    finally:
        canopy.set_wait_bound(-1)
    assert prev == 1 << 24
    return out


def _heavy_chain_nodes(par):
    """Nodes on the heavy chains that start at a root (the chains that wait for nothing): the
    heavy child is the child with the largest subtree, the lowest id on ties."""
    T = len(par)
    size = np.ones(T, int)
    for i in range(T - 1, 0, -1):
        if par[i] >= 0:
            size[par[i]] += size[i]
    keep = set()
    for r in np.nonzero(par < 0)[0]:
        n = int(r)
        while n >= 0:
            keep.add(n)
            kids = [c for c in range(T) if par[c] == n]
            n = max(kids, key=lambda c: (size[c], -c)) if kids else -1
    return keep


@pytest.mark.parametrize("T,tree,waves", [(64, "skewed", 0), (48, "random", 0), (128, "random", 1),
                                          (256, "random", 2)])
def test_lost_handoff_in_the_sub_block_chain(canopy, T, tree, waves):
    """17-64 nodes (the 17-64 kernel) and 65-256 nodes (the wave-per-sub-block kernel): the
    first 16-node sub-block waits for nothing, every later one waits for its predecessors."""
    import torch
    B, H = 1, 2
    inp = synth.make_inputs(B, H, T, tree=tree, dtype="bf16", seed=900 + T)
    d = to_device(inp)
    _say("lost hand-off, sub-block chain", T, tree, waves)

    def run():
        out = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                                 waves=waves, structure=True)
        torch.cuda.synchronize()
        return out
    O, U, ell, mask, depth, st = _with_bound_zero(canopy, run)
    assert st.cpu().numpy().tolist() == [-2] * B
    O, U = O.cpu().numpy(), U.cpu().numpy()
    assert np.isnan(O[:, 16:]).all() and np.isnan(U[:, 16:]).all()
    ref = run_oracle(inp)
    assert_close_heads("O rows 0-15", O[:, :16], ref["O"][:, :16], TOL["bf16"])
    assert_close_heads("U rows 0-15", U[:, :16], ref["U"][:, :16], TOL["bf16"])
    # the default bound again: the same call is whole
    O, U, ell, mask, depth, st = run()
    assert st.cpu().numpy().tolist() == [0] * B
    assert_close_heads("O", O.cpu().numpy(), ref["O"], TOL["bf16"])
    assert_close_heads("U", U.cpu().numpy(), ref["U"], TOL["bf16"])


@pytest.mark.parametrize("T,tree,dtype", [(16, "topk", "bf16"), (40, "random", "fp32")])
def test_lost_handoff_in_the_hybrid(canopy, T, tree, dtype):
    """The chain hybrid: chains that start from a fork snapshot give up; the heavy chain from
    the root keeps its values, and every node of a lost chain, and of the chains forking off
    it, is NaN."""
    import torch
    B, H = 1, 2
    kw = {"branching": (3, 4)} if tree == "topk" else {}
    inp = synth.make_inputs(B, H, T, tree=tree, dtype=dtype, seed=950 + T, tree_kw=kw)
    d = to_device(inp)
    _say("lost hand-off, hybrid", T, tree, dtype)

    def run():
        O, U, snap, st = canopy.hybrid_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                              d["parent"])
        torch.cuda.synchronize()
        return O.cpu().numpy(), U.cpu().numpy(), st.cpu().numpy()
    O, U, st = _with_bound_zero(canopy, run)
    assert st.tolist() == [-2] * B
    keep = sorted(_heavy_chain_nodes(inp["parent"][0]))
    lost = sorted(set(range(T)) - set(keep))
    assert lost, "the tree has no light chain"
    assert np.isnan(O[:, lost]).all() and np.isnan(U[:, lost]).all()
    ref = run_oracle(inp)
    assert_close_heads("O heavy chain", O[:, keep], ref["O"][:, keep], TOL[dtype])
    assert_close_heads("U heavy chain", U[:, keep], ref["U"][:, keep], TOL[dtype])
    O, U, st = run()
    assert st.tolist() == [0] * B
    assert_close_heads("O", O, ref["O"], TOL[dtype])
    assert_close_heads("U", U, ref["U"], TOL[dtype])
