"""The tree closed form in NumPy, for the tests only.

It restates, per node, the algebra that the HIP library implements (the canopy project page,
"The tree closed form" and "Design decisions / Two solve strategies"), so that the tests can
(1) pin the oracle against a second formulation that shares nothing with it and (2) check every
solve strategy against the oracle before any kernel runs. It is neither the oracle nor the
product, and imports neither.

The matrices are built entry by entry from each node's root path: node i's row holds one entry
per node j on path(i), weighted by the decay accumulated strictly below j on that path
(exp(l_i - l_j), with l the running sum of log alpha from the root). The G row leaves out i
itself and carries beta_i; the C row keeps it. The right-hand side subtracts the decayed
initial state's read of k_i, and the output starts from its read of q_i. The commit replays the
accepted path's updates, S <- alpha_n S + k_n u_n^T, root first.
"""
from __future__ import annotations

import numpy as np


def root_paths(parent):
    """path(i) for every node, as a list of node ids from the root down to i (a node's list is
    its parent's list with itself appended)."""
    paths = []
    for i, p in enumerate(np.asarray(parent)):
        paths.append((paths[p] + [i]) if p >= 0 else [i])
    return paths


def depth_of(parent):
    """|A(i)|: the length of each node's root path, minus the node."""
    return np.array([len(p) - 1 for p in root_paths(parent)], dtype=int)


def log_decay(parent, alpha, dtype=np.float64):
    """l_i: log alpha summed along path(i), root first, in ``dtype``."""
    la = np.log(np.asarray(alpha, dtype=dtype))
    ell = np.empty(len(parent), dtype=dtype)
    for i, path in enumerate(root_paths(parent)):
        acc = dtype(0)
        for n in path:
            acc = acc + la[n]
        ell[i] = acc
    return ell


def build_system(parent, q, k, v, alpha, beta, S0, dtype=np.float64, naive_ratio=False,
                 drop=None):
    """G, C, R, the output's first term and l for one (batch, head), each row from the node's
    root path.

    ``naive_ratio`` weighs an entry by the ratio of cumulative decays P_i / P_j instead of
    exp(l_i - l_j) (a negative control). ``drop`` plants one of the mistakes of the
    feature-drop controls: "causal" (every earlier node counted as an ancestor, the causal
    triangle), "gamma" (no decay weight), "strict_c" (C without the node's own entry), "chain"
    (the tree read as a chain)."""
    q, k, v = (np.asarray(x, dtype=dtype) for x in (q, k, v))
    beta = np.asarray(beta, dtype=dtype)
    S0 = np.asarray(S0, dtype=dtype)
    T = len(parent)
    par = np.arange(-1, T - 1) if drop == "chain" else np.asarray(parent)
    ell = log_decay(par, alpha, dtype)
    P = np.exp(ell)
    rows = [list(range(i + 1)) for i in range(T)] if drop == "causal" else root_paths(par)
    G = np.zeros((T, T), dtype=dtype)
    C = np.zeros((T, T), dtype=dtype)
    one = dtype(1)
    with np.errstate(all="ignore"):
        for i in range(T):
            for j in rows[i]:
                if drop == "gamma":
                    w = one
                elif naive_ratio:
                    w = P[i] / P[j]
                else:
                    w = np.exp(ell[i] - ell[j])
                if j != i:
                    G[i, j] = beta[i] * w * np.dot(k[i], k[j])
                if j != i or drop != "strict_c":
                    C[i, j] = w * np.dot(q[i], k[j])
    R = np.empty((T, v.shape[1]), dtype=dtype)
    O0 = np.empty((T, S0.shape[1]), dtype=dtype)
    for i in range(T):
        R[i] = beta[i] * (v[i] - P[i] * (S0.T @ k[i]))
        O0[i] = P[i] * (S0.T @ q[i])
    return G, C, R, O0, ell


# ----------------------------------------------------------------------------- solvers
def solve_dense(G, R):
    T = G.shape[0]
    return np.linalg.solve(np.eye(T, dtype=G.dtype) + G, R)


def solve_fwdsub(G, R):
    U = np.array(R, copy=True)
    for i in range(G.shape[0]):
        U[i] = R[i] - G[i, :i] @ U[:i]
    return U


def solve_blocked(G, R, nb=64):
    """Blocked forward substitution: (I + G_bb) U_b = R_b - sum_{c<b} G_bc U_c, the diagonal
    block solved row by row."""
    T = G.shape[0]
    U = np.zeros_like(R)
    for s in range(0, T, nb):
        e = min(T, s + nb)
        rhs = R[s:e] - G[s:e, :s] @ U[:s]
        Gb = G[s:e, s:e]
        for r in range(e - s):
            U[s + r] = rhs[r] - Gb[r, :r] @ U[s:s + r]
    return U


def solve_neumann(G, R, depth):
    """Finite Neumann series: U = sum_{m=0..depth} (-G)^m R."""
    U = np.array(R, copy=True)
    Z = np.array(R, copy=True)
    for _ in range(int(depth)):
        Z = -(G @ Z)
        U = U + Z
    return U


def solve_squaring(G, R, depth):
    """(I+G)^-1 = (I - G)(I + G^2)(I + G^4)... with ceil(log2(depth+1)) factors."""
    nf = int(np.ceil(np.log2(depth + 1))) if depth > 0 else 0
    U = np.array(R, copy=True)
    if nf == 0:
        return U
    Gp = -G
    for _ in range(nf):
        U = U + Gp @ U
        Gp = Gp @ Gp
    return U


def solve_level(G, R, parent):
    """Level-synchronous: for each depth level L in order, U_L = R_L - G_{L,:} U."""
    d = depth_of(parent)
    U = np.zeros_like(R)
    for L in range(int(d.max()) + 1 if len(d) else 0):
        idx = np.nonzero(d == L)[0]
        U[idx] = R[idx] - G[idx] @ U
    return U


SOLVERS = ("dense", "fwdsub", "blocked", "neumann", "squaring", "level")


def closed_form(parent, q, k, v, alpha, beta, S0, solver="dense", dtype=np.float64, **kw):
    """O, U, ell for one (batch, head): q,k [T,dk], v [T,dv], alpha,beta [T], S0 [dk,dv]."""
    G, C, R, O0, ell = build_system(parent, q, k, v, alpha, beta, S0, dtype=dtype, **kw)
    D = int(depth_of(parent).max()) if len(parent) else 0
    if solver == "dense":
        U = solve_dense(G, R)
    elif solver == "fwdsub":
        U = solve_fwdsub(G, R)
    elif solver == "blocked":
        U = solve_blocked(G, R)
    elif solver == "neumann":
        U = solve_neumann(G, R, D)
    elif solver == "squaring":
        U = solve_squaring(G, R, D)
    elif solver == "level":
        U = solve_level(G, R, parent)
    else:
        raise ValueError(solver)
    return O0 + C @ U, U, ell


def commit_formula(parent, a, k, alpha, U, S0, dtype=np.float64):
    """The state after accepting node a, from the pseudo-values U: the updates of path(a)
    replayed root first, S <- alpha_n S + k_n u_n^T (a < 0: S0 unchanged). Unrolled, this is
    P_a S0 plus each path node's k_j u_j^T decayed by the gates below it."""
    S = np.array(S0, dtype=dtype, copy=True)
    if a < 0:
        return S
    for n in root_paths(parent)[a]:
        S = dtype(alpha[n]) * S + np.outer(np.asarray(k[n], dtype), np.asarray(U[n], dtype))
    return S


def run_batched(inp, solver="dense", dtype=np.float64, **kw):
    """closed_form over every (batch, head) of a synth.make_inputs dict."""
    B, T, H = inp["B"], inp["T"], inp["H"]
    dv = inp["v"].shape[-1]
    O = np.zeros((B, T, H, dv), dtype)
    U = np.zeros((B, T, H, dv), dtype)
    ell = np.zeros((B, T, H), dtype)
    for b in range(B):
        for h in range(H):
            o, u, l = closed_form(inp["parent"][b], inp["q"][b, :, h], inp["k"][b, :, h],
                                  inp["v"][b, :, h], inp["alpha"][b, :, h], inp["beta"][b, :, h],
                                  inp["S0"][b, h], solver=solver, dtype=dtype, **kw)
            O[b, :, h], U[b, :, h], ell[b, :, h] = o, u, l
    return O, U, ell
