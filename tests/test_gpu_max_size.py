"""The largest arrays the ABI accepts in practice: B = 4096 sequences of 256 nodes and 32 heads,
so that q, k, v, O and U hold 2^32 elements each and every index past 2^31 is taken by the
64-bit address arithmetic of the verify kernel AUTO picks there (the blocked solve for two
workgroups per CU: 64-bit bases per (sequence, head), 32-bit offsets within one) and the commit. Inputs are drawn on the
device from a seeded generator (the same distributions as the synthetic recipe: L2-normalized
Gaussian q and k, Gaussian v, sigmoid beta, exp(-softplus) alpha, S0 ~ N(0, 0.1^2), random
recursive trees); the oracle runs on sampled (sequence, head) pairs, the last one included.
About 90 GB of device memory."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, assert_close_heads, assert_close_state

pytestmark = pytest.mark.gpu

B, H, T, D = 4096, 32, 256, 128
SAMPLES = [(0, 0), (B - 1, H - 1), (B // 2, 7), (2047, 31), (2048, 0), (B - 1, 0)]


def _root_path(par, leaf):
    p = [leaf]
    while par[p[-1]] >= 0:
        p.append(int(par[p[-1]]))
    return p[::-1]


def test_index_range_beyond_2_31():
    import torch
    import torch.nn.functional as F
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(4096)
    print("[gpu] max size: drawing inputs", flush=True)
    q = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    S0 = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    step = 256
    for c in range(0, B, step):
        for t in (q, k):
            x = torch.randn((step, T, H, D), generator=g, device=dev)
            t[c:c + step] = (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        v[c:c + step] = torch.randn((step, T, H, D), generator=g, device=dev).to(torch.bfloat16)
        S0[c:c + step] = 0.1 * torch.randn((step, H, D, D), generator=g, device=dev)
    alpha = torch.exp(-F.softplus(torch.randn((B, T, H), generator=g, device=dev)))
    beta = torch.sigmoid(torch.randn((B, T, H), generator=g, device=dev))
    u = torch.rand((B, T), generator=g, device=dev)
    parent = (u * torch.arange(T, device=dev)).floor().to(torch.int32)
    parent[:, 0] = -1
    par_h = parent.cpu().numpy()
    leaves = torch.randint(0, T, (B,), generator=g, device=dev).cpu().numpy()
    path_h = np.full((B, T), -1, np.int32)
    plen_h = np.zeros(B, np.int32)
    for b in range(B):
        p = _root_path(par_h[b], int(leaves[b]))
        path_h[b, :len(p)] = p
        plen_h[b] = len(p)
    path = torch.from_numpy(path_h).to(dev)
    plen = torch.from_numpy(plen_h).to(dev)
    torch.cuda.synchronize()
    assert q.numel() == 2 ** 32

    print("[gpu] max size: verify and commit", flush=True)
    O, U, ell, mask, depth, st = tsv.tree_verify(q, k, v, alpha, beta, S0, parent, structure=True)
    S_new, pst = tsv.commit(S0, k, U, alpha, parent, path, plen)
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0 and int(pst.abs().sum()) == 0

    for b, h in SAMPLES:
        print("[gpu] max size: oracle on", b, h, flush=True)
        one = lambda t: t[b:b + 1, :, h:h + 1].float().cpu().numpy().astype(np.float64)
        ins = dict(q=one(q), k=one(k), v=one(v), alpha=alpha[b:b + 1, :, h:h + 1].cpu().numpy().astype(np.float64),
                   beta=beta[b:b + 1, :, h:h + 1].cpu().numpy().astype(np.float64),
                   S0=S0[b:b + 1, h:h + 1].cpu().numpy().astype(np.float64))
        ref = oracle.gdn_tree(par_h[b:b + 1], ins["q"], ins["k"], ins["v"], ins["alpha"], ins["beta"], ins["S0"])
        assert_close_heads(f"O[{b},{h}]", O[b:b + 1, :, h:h + 1].cpu().numpy(), ref["O"], TOL["bf16"])
        assert_close_heads(f"U[{b},{h}]", U[b:b + 1, :, h:h + 1].cpu().numpy(), ref["U"], TOL["bf16"])
        S_ref, st_ref = oracle.commit(par_h[b:b + 1], path_h[b:b + 1], plen_h[b:b + 1], ins["k"], ins["v"],
                                      ins["alpha"], ins["beta"], ins["S0"])
        assert st_ref.tolist() == [0]
        assert_close_state(f"S_new[{b},{h}]", S_new[b:b + 1, h:h + 1].cpu().numpy(), S_ref, TOL["bf16"])
        dep_ref, mask_ref, _ = oracle.tree_structure(par_h[b:b + 1])
        assert np.array_equal(depth[b:b + 1].cpu().numpy(), dep_ref)
        assert np.array_equal(mask[b:b + 1].cpu().numpy().view(np.uint32), mask_ref)
    del q, k, v, S0, O, U, S_new
    torch.cuda.empty_cache()
