"""NumPy prototype of the tree closed form, used by the tests only.

It states the algebra that the HIP library implements, written from the canopy project page
("The tree closed form" and "Design decisions / Two solve strategies"), so that the tests can
(1) pin the oracle against an independent formula and (2) check every solve strategy against
the oracle before any kernel runs. It is not the oracle and not the product: it imports
neither.

For one (batch, head) with T nodes (parents before children):
  l_i = log alpha_i + l_parent(i)                 (0 for a root's parent)
  Gamma_ij = exp(l_i - l_j) for j in path(i), else 0
  G_ij = beta_i Gamma_ij k_i.k_j for j a strict ancestor of i, else 0
  R_i = beta_i (v_i - exp(l_i) S0^T k_i)
  (I + G) U = R
  C_ij = Gamma_ij q_i.k_j for j in path(i), else 0
  O = diag(exp l) Q S0 + C U
  S_a = exp(l_a) S0 + sum_{j in path(a)} Gamma_aj k_j u_j^T
"""
from __future__ import annotations

import numpy as np


def ancestor_masks(parent):
    """Strict and inclusive ancestor masks (bool [T,T]) by walking parents."""
    T = len(parent)
    Mp = np.zeros((T, T), dtype=bool)
    for i in range(T):
        n = i
        while n >= 0:
            Mp[i, n] = True
            n = parent[n]
    Mm = Mp & ~np.eye(T, dtype=bool)
    return Mm, Mp


def depth_of(parent):
    Mm, _ = ancestor_masks(parent)
    return Mm.sum(1)


def log_decay(parent, alpha, dtype=np.float64):
    la = np.log(np.asarray(alpha, dtype=dtype))
    ell = np.zeros(len(parent), dtype=dtype)
    for i in range(len(parent)):
        ell[i] = la[i] + (ell[parent[i]] if parent[i] >= 0 else dtype(0))
    return ell


def build_system(parent, q, k, v, alpha, beta, S0, dtype=np.float64, naive_ratio=False,
                 drop=None):
    """G, C, R, the output's first term and ell for one (batch, head).

    ``naive_ratio`` forms Gamma as P_i / P_j instead of exp(l_i - l_j) (a negative control).
    ``drop`` plants one of the feature-drop mistakes used by the control tests:
    "causal" (lower triangle instead of the ancestor mask), "gamma" (no decay ratio in G, C),
    "strict_c" (C without its diagonal), "chain" (the tree read as a chain)."""
    q, k, v = (np.asarray(x, dtype=dtype) for x in (q, k, v))
    beta = np.asarray(beta, dtype=dtype)
    S0 = np.asarray(S0, dtype=dtype)
    par = np.asarray(parent)
    if drop == "chain":
        par = np.arange(-1, len(par) - 1)
    Mm, Mp = ancestor_masks(par)
    if drop == "causal":
        T = len(par)
        Mp = np.tril(np.ones((T, T), dtype=bool))
        Mm = Mp & ~np.eye(T, dtype=bool)
    ell = log_decay(par, alpha, dtype)
    P = np.exp(ell)
    if naive_ratio:
        with np.errstate(all="ignore"):
            Gam = np.where(Mp, P[:, None] / P[None, :], 0.0).astype(dtype)
    else:
        diff = np.where(Mp, ell[:, None] - ell[None, :], 0.0)
        Gam = np.where(Mp, np.exp(diff), 0.0).astype(dtype)
    if drop == "gamma":
        Gam = Mp.astype(dtype)
    G = beta[:, None] * Gam * (k @ k.T) * Mm
    Mc = Mm if drop == "strict_c" else Mp
    C = Gam * (q @ k.T) * Mc
    R = beta[:, None] * (v - P[:, None] * (k @ S0))
    O0 = P[:, None] * (q @ S0)
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
    """S_a = exp(l_a) S0 + sum_{j in path(a)} Gamma_aj k_j u_j^T (a < 0: S0)."""
    S0 = np.asarray(S0, dtype=dtype)
    if a < 0:
        return S0.copy()
    ell = log_decay(parent, alpha, dtype)
    S = np.exp(ell[a]) * S0
    j = a
    while j >= 0:
        S = S + np.exp(ell[a] - ell[j]) * np.outer(np.asarray(k[j], dtype), np.asarray(U[j], dtype))
        j = parent[j]
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
