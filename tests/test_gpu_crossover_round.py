"""Rounds of the crossover's parallel path (stacked GDN layers on one tree: every layer's tree
verify from its own state, then one launch committing the accepted path in every layer) against
the oracle, at the crossover's smallest and largest cells.

- Smallest: a 3-node chain, B=1, H=32, 24 layers, two chained rounds (the second verifies from
  the states the first committed).
- Largest: width 16, T=256 (depth 16), B=16, H=32, one round. Its inputs come from the seeded
  generators at about 2.6 s per layer on the host, so 6 layers stand in for the crossover's 24:
  the layered commit is the same launch for any layer count up to 64.

Every layer's O and U against the oracle's per-path recurrence from that layer's state, and
every committed state against the oracle's path commit (max per-(batch, head) relative error
2e-3, bf16 q/k/v with fp32 state; path status bit-exact)."""
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


@pytest.mark.parametrize("W,T,B,L,rounds", [(1, 3, 1, 24, 2), (16, 256, 16, 6, 1)])
def test_crossover_rounds(canopy, W, T, B, L, rounds):
    import torch
    par = synth.level_tree(T, W)
    layers = [synth.make_inputs(B, 32, T, dtype="bf16", seed=9100 + 31 * T + l, parents=par) for l in range(L)]
    ds = [to_device(x) for x in layers]
    parent = ds[0]["parent"]
    S = [d["S0"].clone() for d in ds]
    S_ref = [x["S0"].astype(np.float64) for x in layers]
    rng = np.random.default_rng(9200 + T)
    for r in range(rounds):
        path = np.full((B, T), -1, np.int32)
        plen = np.zeros((B,), np.int32)
        for b in range(B):
            p = synth.random_leaf_path(par, rng)
            path[b, :len(p)] = p
            plen[b] = len(p)
        _say("crossover round", W, T, B, L, r)
        Us, outs = [], []
        for l, d in enumerate(ds):
            O, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S[l], parent)
            Us.append(U)
            outs.append(O)
        S, st = canopy.commit_layers(S, [d["k"] for d in ds], Us, [d["alpha"] for d in ds], parent,
                                     torch.from_numpy(path).cuda(), torch.from_numpy(plen).cuda())
        torch.cuda.synchronize()
        assert st.cpu().numpy().tolist() == [0] * B
        for l, x in enumerate(layers):
            ref = oracle.gdn_tree(x["parent"], x["q"], x["k"], x["v"], x["alpha"], x["beta"], S_ref[l])
            assert_close_heads(f"O layer {l}", outs[l].cpu().numpy(), ref["O"], TOL["bf16"])
            assert_close_heads(f"U layer {l}", Us[l].cpu().numpy(), ref["U"], TOL["bf16"])
            S_next, pst = oracle.commit(x["parent"], path, plen, x["k"], x["v"], x["alpha"], x["beta"], S_ref[l])
            assert pst.tolist() == [0] * B
            assert_close_state(f"S_new layer {l}", S[l].cpu().numpy(), S_next, TOL["bf16"])
            S_ref[l] = S_next
