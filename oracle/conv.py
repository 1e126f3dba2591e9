"""Oracle for the root-path causal convolution of a draft tree: test infrastructure only.

Before a Gated DeltaNet layer, a short causal convolution (kernel size 4 in the canopy page's
model, "Qwen3.5-9B shapes") mixes each token's projected inputs with those of the tokens before
it. On a draft tree a node's "tokens before it" are its root path, and for positions before the
root the convolution reads the committed convolution state; after verification the state is
rolled forward along the accepted path (the canopy page, "M7 ...", stretch item: the
convolution "must also follow each node's root path, and commit must update the convolution
state with the accepted tokens").

Plain NumPy in fp64, one node and one window position at a time. Shapes:
    x      [B,T,C]      inputs of every node (padding rows past tree_len ignored)
    w      [C,K]        depthwise weights; w[c, K-1] multiplies the node itself
    state  [B,K-1,C]    the K-1 committed inputs before the tree, oldest first
    parent [B,T]; tree_len [B] or None.
"""
from __future__ import annotations

import numpy as np


def _window_row(parent, x_b, state_b, i, back):
    """The input `back` positions before node i on its root path (back = 0: i itself); before
    the root, row K-1-(back-depth(i)) of the committed state."""
    a = i
    for _ in range(back):
        if a < 0:
            break
        a = parent[a]
        if a < 0:
            break
    if a >= 0:
        return x_b[a]
    # how many steps past the root: depth(i) + 1 steps reach "before the root"
    depth = 0
    j = parent[i]
    while j >= 0:
        depth += 1
        j = parent[j]
    k1 = state_b.shape[0]
    return state_b[k1 - (back - depth)]


def tree_conv(parent, tree_len, x, w, state, silu=False):
    """y[b,i,c] = sum_{j<K} w[c,j] * X(node i, K-1-j positions back) (then SiLU if asked).
    Returns (y [B,T,C] fp64 with NaN on padding rows and malformed trees, status [B]: 0, -1 for
    a length outside 1..T, else 1 + the first node whose parent is outside -1..i-1)."""
    par = np.asarray(parent, np.int64)
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    st = np.asarray(state, np.float64)
    B, T, C = x.shape
    K = w.shape[1]
    assert st.shape == (B, K - 1, C)
    lens = np.full(B, T) if tree_len is None else np.asarray(tree_len, np.int64)
    y = np.full((B, T, C), np.nan)
    status = np.zeros(B, np.int32)
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= T:
            status[b] = -1
            continue
        p = par[b, :n]
        bad = [i for i in range(n) if not (-1 <= p[i] < i)]
        if bad:
            status[b] = bad[0] + 1
            continue
        for i in range(n):
            acc = np.zeros(C)
            for j in range(K):
                acc += w[:, j] * _window_row(p, x[b], st[b], i, K - 1 - j)
            if silu:
                acc = acc / (1.0 + np.exp(-acc))
            y[b, i] = acc
    return y, status


def conv_commit(parent, tree_len, path, path_len, x, state):
    """The convolution state after committing the accepted path: the last K-1 inputs of the
    committed sequence (old state, then the path's nodes), oldest first. Returns (state_new
    [B,K-1,C] fp64, status [B]) with the statuses of the state commit (-1 for path_len or
    tree_len out of range, else 1 + the first position whose node is out of range or not a
    child of the previous one); a bad sequence's state is NaN."""
    par = np.asarray(parent, np.int64)
    pth = np.asarray(path, np.int64)
    plen = np.asarray(path_len, np.int64)
    x = np.asarray(x, np.float64)
    st = np.asarray(state, np.float64)
    B, T, C = x.shape
    K1 = st.shape[1]
    lens = np.full(B, T) if tree_len is None else np.asarray(tree_len, np.int64)
    out = np.full(st.shape, np.nan)
    status = np.zeros(B, np.int32)
    for b in range(B):
        n, m = int(lens[b]), int(plen[b])
        if not 1 <= n <= T or not 0 <= m <= n:
            status[b] = -1
            continue
        s = 0
        for t in range(m):
            node = pth[b, t]
            if not (0 <= node < n) or par[b, node] != (pth[b, t - 1] if t else -1):
                s = t + 1
                break
        status[b] = s
        if s:
            continue
        seq = [st[b, r] for r in range(K1)] + [x[b, pth[b, t]] for t in range(m)]
        for r in range(K1):
            out[b, r] = seq[len(seq) - K1 + r]
    return out, status
