"""Parity of the root-path causal convolution and its state commit against the fp64 oracle
(oracle/conv.py), through the C ABI: fp32 within 1e-6, bf16 within one rounding of the oracle's
value (the kernel accumulates in fp32 and rounds once), padding rows untouched, malformed trees
and paths reported, the commit exact and possible in place."""
import numpy as np
import pytest

import synth
from oracle import conv as oc

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


def _inputs(B, T, C, K, dtype, tree, seed, lens=None):
    rng = np.random.default_rng(seed)
    par = np.full((B, T), -5, np.int32)
    for b in range(B):
        n = T if lens is None else lens[b]
        par[b, :n] = synth.make_tree(tree, n, rng, branching=(3, 4))
    x = rng.standard_normal((B, T, C)).astype(np.float32)
    st = rng.standard_normal((B, K - 1, C)).astype(np.float32)
    w = (rng.standard_normal((C, K)) * 0.5).astype(np.float32)
    if lens is not None:
        for b in range(B):
            x[b, lens[b]:] = np.nan
    if dtype == "bf16":
        xb, sb = synth.bf16_bits(x), synth.bf16_bits(st)
        return par, synth.bf16_widen(xb), synth.bf16_widen(sb), w, xb, sb
    return par, x, st, w, None, None


def _dev(canopy, par, x, st, w, xb, sb, lens):
    import torch
    if xb is not None:
        xd = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
        sd = torch.from_numpy(sb.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        xd, sd = torch.from_numpy(x).cuda(), torch.from_numpy(st).cuda()
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    return xd, sd, torch.from_numpy(w).cuda(), torch.from_numpy(par).cuda(), tl


def _ordered(bits):
    """bf16 bit patterns as integers whose order is the numbers' order (for ulp distances)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)


def _compare(y, ref, dtype, rows):
    if dtype == "fp32":
        den = np.max(np.abs(ref[rows]))
        err = np.max(np.abs(y[rows].astype(np.float64) - ref[rows])) / den
        assert err <= 1e-6, err
    else:
        got = _ordered(y[rows])
        want = _ordered(synth.bf16_bits(ref[rows].astype(np.float32)))
        dist = np.abs(got - want)
        assert dist.max() <= 1, f"{dist.max()} ulp"
        assert (dist == 0).mean() >= 0.99


CASES = [
    (1, 16, 8192, 4, "bf16", True, "topk", None),      # the 9B-shaped layer's channels
    (1, 7, 64, 4, "fp32", False, "binary7", None),
    (3, 100, 256, 3, "bf16", False, "random", [100, 37, 1]),
    (2, 256, 128, 2, "fp32", True, "skewed", None),
    (2, 64, 1024, 4, "fp32", True, "chain", [64, 5]),
]


@pytest.mark.parametrize("B,T,C,K,dtype,silu,tree,lens", CASES)
def test_tree_conv(canopy, B, T, C, K, dtype, silu, tree, lens):
    import torch
    par, x, st, w, xb, sb = _inputs(B, T, C, K, dtype, tree, 70 + T + K, lens)
    xd, sd, wd, pd, tl = _dev(canopy, par, x, st, w, xb, sb, lens)
    _say("tree_conv", B, T, C, K, dtype, silu, tree, lens)
    y = torch.full_like(xd, 3.0)
    y, status = canopy.tree_conv(xd, wd, sd, pd, silu=silu, tree_len=tl, out=y)
    torch.cuda.synchronize()
    ref, st_ref = oc.tree_conv(par, lens, x, w, st, silu=silu)
    assert status.cpu().numpy().tolist() == st_ref.tolist() == [0] * B
    yh = y.cpu()
    yb = yh.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else yh.numpy()
    for b in range(B):
        n = T if lens is None else lens[b]
        _compare(yb[b], ref[b], dtype, slice(0, n))
        pad = yh[b, n:].float().numpy()
        assert (pad == 3.0).all(), "padding rows written"


def test_tree_conv_malformed_tree(canopy):
    import torch
    B, T, C, K = 2, 20, 64, 4
    par, x, st, w, xb, sb = _inputs(B, T, C, K, "fp32", "random", 91)
    par[1, 13] = 15
    xd, sd, wd, pd, tl = _dev(canopy, par, x, st, w, xb, sb, None)
    y, status = canopy.tree_conv(xd, wd, sd, pd)
    torch.cuda.synchronize()
    ref, st_ref = oc.tree_conv(par, None, x, w, st)
    assert status.cpu().numpy().tolist() == st_ref.tolist() == [0, 14]
    assert np.isnan(y[1].cpu().numpy()).all()
    _compare(y[0].cpu().numpy(), ref[0], "fp32", slice(0, T))


@pytest.mark.parametrize("dtype,K", [("bf16", 4), ("fp32", 3), ("bf16", 2)])
def test_conv_commit(canopy, dtype, K):
    """Random leaf paths, a one-node path (the old state shifts), an empty path, a broken path
    and a path longer than its ragged sequence; then the same commit in place."""
    import torch
    B, T, C = 5, 30, 512
    lens = [30, 30, 30, 30, 4]
    par, x, st, w, xb, sb = _inputs(B, T, C, K, dtype, "random", 92 + K, lens)
    rng = np.random.default_rng(5)
    path = np.full((B, T), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in (0, 4):
        p = synth.random_leaf_path(par[b, :lens[b]], rng)
        path[b, :len(p)] = p
        plen[b] = len(p)
    path[1, 0], plen[1] = 0, 1
    plen[2] = 0
    path[3, :3], plen[3] = [0, 5, 2], 3
    if plen[4] < 5:
        path[4, :5], plen[4] = [0, 1, 2, 3, 4], 5         # longer than the 4-node tree
    xd, sd, wd, pd, tl = _dev(canopy, par, x, st, w, xb, sb, lens)
    paths, plens = torch.from_numpy(path).cuda(), torch.from_numpy(plen).cuda()
    _say("conv_commit", dtype, K)
    new, status = canopy.conv_commit(xd, sd, pd, paths, plens, tree_len=tl)
    torch.cuda.synchronize()
    ref, st_ref = oc.conv_commit(par, lens, path, plen, x, st)
    got_status = status.cpu().numpy().tolist()
    assert got_status == st_ref.tolist()
    assert st_ref[0] == 0 and st_ref[1] == 0 and st_ref[2] == 0 and st_ref[3] > 0 and st_ref[4] == -1
    got = new.float().cpu().numpy()
    ok = st_ref == 0
    assert np.array_equal(got[ok], ref[ok].astype(np.float32))
    assert np.isnan(got[~ok]).all()
    inplace = sd.clone()
    new2, _ = canopy.conv_commit(xd, inplace, pd, paths, plens, tree_len=tl, out=inplace)
    torch.cuda.synchronize()
    okd = torch.from_numpy(ok).cuda()
    assert torch.equal(new2[okd], new[okd])
