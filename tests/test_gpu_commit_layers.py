"""One launch for every layer's commit: bit for bit the per-layer commits, and the oracle's
states, including grouped heads, a ragged batch, in-place commits and path errors."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close_state, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


def _layers(L, B, H, T, seed, HK=None, lens=None, tree="random"):
    """L layers on one tree and path: each with its own draws (seed + l)."""
    base = synth.make_inputs(B, H, T, tree=tree, dtype="bf16", seed=seed, HK=HK, tree_len=lens)
    out = []
    for l in range(L):
        inp = synth.make_inputs(B, H, T, dtype="bf16", seed=seed + 1 + l, HK=HK, tree_len=lens,
                                parents=base["parent"])
        inp["path"], inp["path_len"] = base["path"], base["path_len"]
        inp["parent"] = base["parent"]
        out.append(inp)
    return out


@pytest.mark.parametrize("L,B,H,T,HK,lens", [(1, 1, 4, 16, None, None), (3, 2, 4, 64, 2, None),
                                             (24, 1, 32, 16, None, None), (5, 3, 4, 100, 2, [100, 40, 1])])
def test_commit_layers_match_per_layer(canopy, L, B, H, T, HK, lens):
    import torch
    layers = _layers(L, B, H, T, 800 + T + L, HK=HK, lens=lens)
    ds = [to_device(x) for x in layers]
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    Us = []
    for d in ds:
        _, U, _ = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"],
                                     tree_len=tl)
        Us.append(U)
    d0 = ds[0]
    print("[gpu] commit_layers", L, B, H, T, HK, lens, flush=True)
    outs, st = canopy.commit_layers([d["S0"] for d in ds], [d["k"] for d in ds], Us,
                                    [d["alpha"] for d in ds], d0["parent"], d0["path"], d0["path_len"],
                                    tree_len=tl)
    singles = [canopy.commit(d["S0"], d["k"], U, d["alpha"], d0["parent"], d0["path"], d0["path_len"],
                             tree_len=tl) for d, U in zip(ds, Us)]
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0] * B
    for l in range(L):
        assert torch.equal(outs[l], singles[l][0]), f"layer {l}"
    for l in (0, L - 1):
        x = layers[l]
        S_ref, st_ref = oracle.commit_ragged(x["parent"], x["tree_len"], x["path"], x["path_len"], x["k"],
                                             x["v"], x["alpha"], x["beta"], x["S0"])
        assert_close_state(f"layer {l}", outs[l].cpu().numpy(), S_ref, TOL["bf16"])


def test_commit_layers_in_place_and_bad_path(canopy):
    import torch
    L, B, H, T = 4, 3, 2, 30
    layers = _layers(L, B, H, T, 870, tree="chain")
    layers[0]["path"][2, :3] = [0, 2, 1]          # broken at position 1
    layers[0]["path_len"][2] = 3
    ds = [to_device(x) for x in layers]
    Us = [canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])[1]
          for d in ds]
    d0 = ds[0]
    ref, st_ref = canopy.commit_layers([d["S0"] for d in ds], [d["k"] for d in ds], Us,
                                       [d["alpha"] for d in ds], d0["parent"], d0["path"], d0["path_len"])
    S = [d["S0"].clone() for d in ds]
    outs, st = canopy.commit_layers(S, [d["k"] for d in ds], Us, [d["alpha"] for d in ds], d0["parent"],
                                    d0["path"], d0["path_len"], outs=S)
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == st_ref.cpu().numpy().tolist() == [0, 0, 2]
    for l in range(L):
        assert torch.equal(outs[l][:2], ref[l][:2])
        assert torch.isnan(outs[l][2]).all()


def test_serial_commit_layers(canopy):
    import torch
    L, B, H, T = 3, 2, 2, 20
    layers = _layers(L, B, H, T, 880)
    ds = [to_device(x) for x in layers]
    snaps = [canopy.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"])[2]
             for d in ds]
    d0 = ds[0]
    outs, st = canopy.serial_commit_layers(snaps, [d["S0"] for d in ds], d0["parent"], d0["path"],
                                           d0["path_len"])
    singles = [canopy.serial_commit(sn, d["S0"], d0["parent"], d0["path"], d0["path_len"])[0]
               for sn, d in zip(snaps, ds)]
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0, 0]
    for l in range(L):
        assert torch.equal(outs[l], singles[l])
