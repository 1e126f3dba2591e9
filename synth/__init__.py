"""Seeded synthetic inputs for tree-structured Gated DeltaNet verification.

This module is shared by the tests, the benchmark and the oracle's callers. It holds no part
of the method's arithmetic: it only draws trees (parent arrays), activations, gates and the
committed state, and picks accepted paths. Nothing here imports the oracle or the HIP library.

Shapes and distributions follow the workload descriptions used for this operator (the canopy
project page, "Qwen3.5-9B shapes" and "Benchmarks"): per head a 128 x 128 state, L2-normalised
Gaussian queries and keys, standard normal values, beta = sigmoid(N(0,1)),
alpha = exp(-softplus(N(0,1))), S0 ~ N(0, 0.1^2). Every draw comes from one
``numpy.random.default_rng(seed)`` in a fixed order: tree, x_q, x_k, v, beta logits,
alpha logits, S0, then the accepted paths. Draws are fp64, stored as fp32; bf16 inputs are
rounded to nearest-even from the fp32 value.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "chain", "star", "binary7", "topk_tree", "skewed_tree", "random_tree", "level_tree",
    "make_tree", "tree_depths", "children_of", "leaves", "root_path", "random_leaf_path",
    "dfs_preorder", "level_order", "relabel", "bf16_bits", "bf16_widen", "make_inputs",
]


# --------------------------------------------------------------------------- tree families
def chain(T: int) -> np.ndarray:
    """A chain 0 -> 1 -> ... -> T-1 (depth T-1)."""
    p = np.arange(-1, T - 1, dtype=np.int32)
    return p


def star(T: int) -> np.ndarray:
    """A root with T-1 children (depth 1)."""
    p = np.zeros(T, dtype=np.int32)
    p[0] = -1
    return p


def binary7() -> np.ndarray:
    """The balanced binary tree of 7 nodes in level order."""
    return np.array([-1, 0, 0, 1, 1, 2, 2], dtype=np.int32)


def topk_tree(branching) -> np.ndarray:
    """Balanced tree in level order: the root, then ``branching[0]`` children of the root, then
    ``branching[1]`` children of every node of level 1, and so on. ``(3, 4)`` gives 1+3+12."""
    parents = [-1]
    level = [0]
    for b in branching:
        nxt = []
        for node in level:
            for _ in range(b):
                parents.append(node)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.array(parents, dtype=np.int32)


def skewed_tree(T: int, rng: np.random.Generator, p_chain: float = 0.7) -> np.ndarray:
    """Node i's parent is i-1 with probability ``p_chain``, else uniform over 0..i-1."""
    p = np.empty(T, dtype=np.int32)
    p[0] = -1
    for i in range(1, T):
        if rng.random() < p_chain:
            p[i] = i - 1
        else:
            p[i] = rng.integers(0, i)
    return p


def random_tree(T: int, rng: np.random.Generator) -> np.ndarray:
    """Random recursive tree: node i's parent is uniform over 0..i-1."""
    p = np.empty(T, dtype=np.int32)
    p[0] = -1
    for i in range(1, T):
        p[i] = rng.integers(0, i)
    return p


def level_tree(T: int, W: int) -> np.ndarray:
    """Depth x width family: a root, then levels of W nodes (the last one partial). Node j of a
    level takes as parent node (j mod n_prev) of the level above. W = 1 is a chain; W >= T-1 is
    a star."""
    p = [-1]
    prev = [0]
    nxt_id = 1
    while nxt_id < T:
        n = min(W, T - nxt_id)
        cur = []
        for j in range(n):
            p.append(prev[j % len(prev)])
            cur.append(nxt_id)
            nxt_id += 1
        prev = cur
    return np.array(p, dtype=np.int32)


def make_tree(kind: str, T: int, rng: np.random.Generator | None = None, **kw) -> np.ndarray:
    if kind == "chain":
        return chain(T)
    if kind == "star":
        return star(T)
    if kind == "binary7":
        assert T == 7
        return binary7()
    if kind == "topk":
        p = topk_tree(kw["branching"])
        assert len(p) == T, (len(p), T)
        return p
    if kind == "skewed":
        return skewed_tree(T, rng, kw.get("p_chain", 0.7))
    if kind == "random":
        return random_tree(T, rng)
    if kind == "level":
        return level_tree(T, kw["width"])
    raise ValueError(f"unknown tree kind {kind!r}")


# --------------------------------------------------------------------------- tree helpers
def children_of(parent) -> list:
    T = len(parent)
    ch = [[] for _ in range(T)]
    for i in range(T):
        if parent[i] >= 0:
            ch[parent[i]].append(i)
    return ch


def tree_depths(parent) -> np.ndarray:
    """Number of strict ancestors of every node (parent[i] < i assumed)."""
    d = np.zeros(len(parent), dtype=np.int32)
    for i in range(len(parent)):
        d[i] = 0 if parent[i] < 0 else d[parent[i]] + 1
    return d


def leaves(parent) -> np.ndarray:
    ch = children_of(parent)
    return np.array([i for i in range(len(parent)) if not ch[i]], dtype=np.int32)


def root_path(parent, a: int) -> np.ndarray:
    """Node ids from the root down to ``a`` (root first)."""
    out = []
    while a >= 0:
        out.append(a)
        a = parent[a]
    return np.array(out[::-1], dtype=np.int32)


def random_leaf_path(parent, rng: np.random.Generator) -> np.ndarray:
    lv = leaves(parent)
    a = int(lv[rng.integers(0, len(lv))])
    return root_path(parent, a)


def dfs_preorder(parent) -> np.ndarray:
    """A DFS pre-order of the nodes (children visited in increasing id)."""
    ch = children_of(parent)
    roots = [i for i in range(len(parent)) if parent[i] < 0]
    order, stack = [], list(reversed(roots))
    while stack:
        n = stack.pop()
        order.append(n)
        stack.extend(reversed(ch[n]))
    return np.array(order, dtype=np.int32)


def level_order(parent) -> np.ndarray:
    """Nodes sorted by depth (stable in id)."""
    d = tree_depths(parent)
    return np.argsort(d, kind="stable").astype(np.int32)


def relabel(parent, order):
    """Renumber nodes so that new node n is old node ``order[n]``. ``order`` must be topological.
    Returns the new parent array."""
    order = np.asarray(order)
    T = len(order)
    new_of_old = np.empty(T, dtype=np.int64)
    new_of_old[order] = np.arange(T)
    newp = np.empty(T, dtype=np.int32)
    for n in range(T):
        po = parent[order[n]]
        newp[n] = -1 if po < 0 else new_of_old[po]
    assert all(newp[n] < n for n in range(T)), "order is not topological"
    return newp


# --------------------------------------------------------------------------- bf16 rounding
def bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_widen(bits) -> np.ndarray:
    """Exact fp32 value of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# --------------------------------------------------------------------------- inputs
def _l2n(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_inputs(B: int, H: int, T: int, *, tree: str = "random", dtype: str = "bf16",
                seed: int = 0, dk: int = 128, dv: int = 128, tree_kw: dict | None = None,
                parents=None, s0_std: float = 0.1, HK: int | None = None, tree_len=None,
                pad: float = float("nan")) -> dict:
    """Draw one layer's inputs.

    ``tree`` names a family of ``make_tree``; for random families every batch element gets its
    own tree. ``parents`` (a [B,T] array or one [T] array) overrides the drawn trees. Returns a
    dict with fp32 arrays q, k [B,T,HK,d], v [B,T,H,d], alpha, beta [B,T,H], S0 [B,H,dk,dv],
    parent [B,T] int32, a random root-to-leaf path per sequence (``path`` [B,T] root first,
    padded with -1, and ``path_len`` [B]), and for bf16 inputs the 16-bit patterns q_bits,
    k_bits, v_bits. q, k, v hold exactly the values the device reads (already rounded for bf16).

    ``HK`` (default H) is the number of q/k heads, a divisor of the H value heads. ``tree_len``
    ([B] ints in 1..T) makes a ragged batch: sequence b's tree has tree_len[b] nodes, and the
    rows past it are padding, filled with ``pad`` (q, k, v, alpha, beta) and with parents that
    are not valid (-5).
    """
    rng = np.random.default_rng(seed)
    tree_kw = tree_kw or {}
    HK = H if HK is None else HK
    assert H % HK == 0
    lens = None if tree_len is None else np.asarray(tree_len, dtype=np.int32)
    if parents is not None:
        par = np.asarray(parents, dtype=np.int32)
        if par.ndim == 1:
            par = np.broadcast_to(par, (B, T)).copy()
    elif lens is None:
        par = np.stack([make_tree(tree, T, rng, **tree_kw) for _ in range(B)]).astype(np.int32)
    else:
        par = np.full((B, T), -5, dtype=np.int32)
        for b in range(B):
            par[b, :lens[b]] = make_tree(tree, int(lens[b]), rng, **tree_kw)
    assert par.shape == (B, T)
    xq = rng.standard_normal((B, T, HK, dk))
    xk = rng.standard_normal((B, T, HK, dk))
    v = rng.standard_normal((B, T, H, dv))
    zb = rng.standard_normal((B, T, H))
    za = rng.standard_normal((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv)) * s0_std
    q = _l2n(xq).astype(np.float32)
    k = _l2n(xk).astype(np.float32)
    v = v.astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    alpha = np.exp(-np.logaddexp(0.0, za)).astype(np.float32)
    S0 = S0.astype(np.float32)
    paths = np.full((B, T), -1, dtype=np.int32)
    plen = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = T if lens is None else int(lens[b])
        pth = random_leaf_path(par[b, :n], rng)
        paths[b, :len(pth)] = pth
        plen[b] = len(pth)
    if lens is not None:
        for b in range(B):
            n = int(lens[b])
            for arr in (q, k, v, alpha, beta):
                arr[b, n:] = pad
    out = dict(B=B, H=H, HK=HK, T=T, dk=dk, dv=dv, dtype=dtype, parent=par, alpha=alpha,
               beta=beta, S0=S0, path=paths, path_len=plen,
               tree_len=None if lens is None else lens.copy())
    if dtype == "bf16":
        for name, arr in (("q", q), ("k", k), ("v", v)):
            bits = bf16_bits(arr)
            out[name + "_bits"] = bits
            out[name] = bf16_widen(bits)
    elif dtype == "fp32":
        out.update(q=q, k=k, v=v)
    else:
        raise ValueError(dtype)
    return out
