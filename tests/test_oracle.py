"""Pins for the oracle (CPU only): hand-derived values, closed forms, invariants, special cases
and brute force, each fixed by the canopy project page or by mathematics rather than by the
oracle itself. The closed-form helper in ``closed_form.py`` is the page's second formulation of
the same quantities ("The tree closed form"), with a library triangular solve."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from _common import elem_rel_err, fro_rel_err, max_rel_err, read_golden, per_head_rel_err, state_rel_err
import closed_form as cf


def _one_head(parent, q, k, v, alpha, beta, S0):
    """Wrap single-(batch, head) arrays into the oracle's [B,T,H,...] layouts."""
    return dict(parent=np.asarray(parent)[None], q=q[None, :, None], k=k[None, :, None],
                v=v[None, :, None], alpha=np.asarray(alpha)[None, :, None],
                beta=np.asarray(beta)[None, :, None], S0=S0[None, None])


def _run(d, **kw):
    return oracle.gdn_tree(d["parent"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], **kw)


# ------------------------------------------------------------------ hand-derived worked example
def test_hand_worked_example():
    g = read_golden("hand_star3_d2.txt")
    par = g["parent"][0].astype(np.int32)
    d = _one_head(par, g["q"][0].reshape(3, 2), g["k"][0].reshape(3, 2), g["v"][0].reshape(3, 2),
                  g["alpha"][0], g["beta"][0], g["S0"][0].reshape(2, 2))
    r = _run(d, all_states=True)
    np.testing.assert_allclose(r["O"][0, :, 0], g["O"][0].reshape(3, 2), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["U"][0, :, 0], g["U"][0].reshape(3, 2), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["ell"][0, :, 0], g["ell_over_log_half"][0] * np.log(0.5),
                               rtol=1e-15, atol=0)
    for n in range(3):
        np.testing.assert_allclose(r["S_all"][0, n, 0], g[f"S_node{n}"][0].reshape(2, 2),
                                   rtol=0, atol=1e-14)
    # commit along each root path reaches the same hand-derived states
    for path, n in (([0], 0), ([0, 1], 1), ([0, 2], 2)):
        pa = np.full((1, 3), -1, np.int32)
        pa[0, :len(path)] = path
        S, st = oracle.commit(d["parent"], pa, [len(path)], d["k"], d["v"], d["alpha"], d["beta"],
                              d["S0"])
        assert st[0] == 0
        np.testing.assert_allclose(S[0, 0], g[f"S_node{n}"][0].reshape(2, 2), rtol=0, atol=1e-14)


def test_hand_single_node_closed_form():
    """T = 1 written out: u0 = b0 (v0 - a0 S0^T k0), o0 = a0 S0^T q0 + (q0.k0) u0."""
    rng = np.random.default_rng(3)
    for dk, dv in ((2, 3), (4, 4), (128, 128)):
        q, k, v = rng.standard_normal((1, dk)), rng.standard_normal((1, dk)), rng.standard_normal((1, dv))
        S0 = rng.standard_normal((dk, dv))
        a, b = 0.7, 0.3
        r = _run(_one_head([-1], q, k, v, [a], [b], S0))
        u0 = b * (v[0] - a * S0.T @ k[0])
        o0 = a * S0.T @ q[0] + (q[0] @ k[0]) * u0
        np.testing.assert_allclose(r["U"][0, 0, 0], u0, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(r["O"][0, 0, 0], o0, rtol=1e-13, atol=1e-13)


def test_hand_two_node_chain_closed_form():
    """T = 2 chain written out with the decayed, rank-1-updated root state."""
    rng = np.random.default_rng(4)
    dk, dv = 3, 2
    q, k, v = rng.standard_normal((2, dk)), rng.standard_normal((2, dk)), rng.standard_normal((2, dv))
    S0 = rng.standard_normal((dk, dv))
    a, b = [0.9, 0.6], [0.5, 0.8]
    r = _run(_one_head([-1, 0], q, k, v, a, b, S0))
    u0 = b[0] * (v[0] - a[0] * S0.T @ k[0])
    S1 = a[0] * S0 + np.outer(k[0], u0)
    u1 = b[1] * (v[1] - a[1] * S1.T @ k[1])
    o1 = a[1] * S1.T @ q[1] + (q[1] @ k[1]) * u1
    np.testing.assert_allclose(r["U"][0, 1, 0], u1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["O"][0, 1, 0], o1, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ tree structure (brute force)
def test_tree_structure_golden():
    g = read_golden("tree_structure.txt")
    for par, dep, msk in zip(g["parent"], g["depth"], g["mask"]):
        depth, mask, st = oracle.tree_structure(par.astype(np.int32))
        assert st[0] == 0
        assert depth[0].tolist() == dep.astype(int).tolist()
        assert mask[0, :, 0].tolist() == msk.astype(np.int64).tolist()


def _closure_mask(parent):
    """Inclusive ancestor relation as the reflexive-transitive closure of the parent relation,
    by repeated boolean squaring (independent of any parent walk)."""
    T = len(parent)
    A = np.eye(T, dtype=np.int64)
    for i in range(T):
        if parent[i] >= 0:
            A[i, parent[i]] = 1
    for _ in range(int(np.ceil(np.log2(max(T, 2)))) + 1):
        A = ((A @ A) > 0).astype(np.int64)
    return A.astype(bool)


@pytest.mark.parametrize("seed", range(6))
def test_mask_depth_vs_closure(seed):
    rng = np.random.default_rng(seed)
    for T in (1, 2, 31, 32, 33, 64, 65, 200, 256):
        kind = ["random", "skewed", "chain", "star"][(seed + T) % 4]
        par = synth.make_tree(kind, T, rng)
        depth, mask, st = oracle.tree_structure(par)
        assert st[0] == 0
        M = _closure_mask(par)
        W = (T + 31) // 32
        bits = np.zeros((T, W * 32), dtype=bool)
        for w in range(W):
            for j in range(32):
                bits[:, w * 32 + j] = (mask[0, :, w] >> j) & 1
        assert np.array_equal(bits[:, :T], M)
        assert not bits[:, T:].any()
        assert np.array_equal(depth[0], M.sum(1) - 1)


def test_invalid_trees_flagged():
    bad = [np.array([0, 0, 1], np.int32),            # node 0 with a parent
           np.array([-1, 0, 2], np.int32),           # self parent
           np.array([-1, 0, 3, 1], np.int32),        # forward parent
           np.array([-1, -2, 0], np.int32)]          # below -1
    expect = [1, 3, 3, 2]
    for par, e in zip(bad, expect):
        _, _, st = oracle.tree_structure(par)
        assert st[0] == e
        T = len(par)
        rng = np.random.default_rng(0)
        d = _one_head(par, rng.standard_normal((T, 4)), rng.standard_normal((T, 4)),
                      rng.standard_normal((T, 4)), np.full(T, 0.5), np.full(T, 0.5),
                      rng.standard_normal((4, 4)))
        r = _run(d)
        assert np.isnan(r["O"]).all() and np.isnan(r["U"]).all()


# ------------------------------------------------------------------ invariants and special cases
def _rand_head(rng, T, dk=128, dv=128, parent=None, kind="random"):
    par = parent if parent is not None else synth.make_tree(kind, T, rng)
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal(T)))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    return par, q, k, v, alpha, beta, S0


def test_chain_equals_product_form():
    """On a chain the tree oracle is the sequential recurrence, written here in the page's
    product form S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t."""
    rng = np.random.default_rng(11)
    T = 40
    par, q, k, v, a, b, S0 = _rand_head(rng, T, parent=synth.chain(T))
    r = _run(_one_head(par, q, k, v, a, b, S0), all_states=True)
    S = S0.copy()
    I = np.eye(128)
    for t in range(T):
        S = a[t] * (I - b[t] * np.outer(k[t], k[t])) @ S + b[t] * np.outer(k[t], v[t])
        np.testing.assert_allclose(r["S_all"][0, t, 0], S, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["O"][0, t, 0], S.T @ q[t], rtol=0, atol=1e-12)


def test_rounds_equal_concatenated_recurrence():
    """Rounds of verify + commit, each on its own tree from the state the previous round
    committed, equal one sequential recurrence over the rounds' accepted tokens in order: the
    final state, and every accepted node's output (the token loop in product form, as above)."""
    rng = np.random.default_rng(17)
    S_chain = 0.1 * rng.standard_normal((128, 128))
    S_rounds = S_chain.copy()
    I = np.eye(128)
    trees = [synth.make_tree("random", 12, rng), synth.topk_tree((3, 4)), synth.chain(5),
             synth.make_tree("skewed", 20, rng)]
    for r, par in enumerate(trees):
        T = len(par)
        _, q, k, v, a, b, _ = _rand_head(rng, T, parent=par)
        d = _one_head(par, q, k, v, a, b, S_rounds)
        out = _run(d)
        path = synth.random_leaf_path(par, rng)
        plen = np.array([len(path)], np.int32)
        pth = np.full((1, T), -1, np.int32)
        pth[0, :len(path)] = path
        S_new, st = oracle.commit(d["parent"], pth, plen, d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
        assert st.tolist() == [0]
        for t in path:  # the round's accepted tokens, root first, through the plain loop
            S_chain = a[t] * (I - b[t] * np.outer(k[t], k[t])) @ S_chain + b[t] * np.outer(k[t], v[t])
            np.testing.assert_allclose(out["O"][0, t, 0], S_chain.T @ q[t], rtol=0, atol=1e-11)
        S_rounds = S_new[0, 0]
        np.testing.assert_allclose(S_rounds, S_chain, rtol=0, atol=1e-11)


def test_beta_zero_decay_only():
    """beta = 0: nothing is written, so o_i = P_i S0^T q_i with P_i the product of alpha along
    path(i), U = 0 and the committed state is P_a S0; with alpha = 1 also, O = Q S0."""
    rng = np.random.default_rng(12)
    T = 30
    par, q, k, v, a, _, S0 = _rand_head(rng, T)
    b = np.zeros(T)
    r = _run(_one_head(par, q, k, v, a, b, S0))
    for i in range(T):
        P = np.prod([a[j] for j in synth.root_path(par, i)])
        np.testing.assert_allclose(r["O"][0, i, 0], P * S0.T @ q[i], rtol=1e-12, atol=1e-14)
    assert np.all(r["U"] == 0)
    leaf = int(synth.leaves(par)[0])
    pth = synth.root_path(par, leaf)
    pa = np.full((1, T), -1, np.int32); pa[0, :len(pth)] = pth
    S, st = oracle.commit(par[None], pa, [len(pth)], k[None, :, None], v[None, :, None],
                          a[None, :, None], b[None, :, None], S0[None, None])
    np.testing.assert_allclose(S[0, 0], np.prod(a[pth]) * S0, rtol=1e-12, atol=1e-15)
    r1 = _run(_one_head(par, q, k, v, np.ones(T), b, S0))
    np.testing.assert_allclose(r1["O"][0, :, 0], q @ S0, rtol=1e-12, atol=1e-14)


def test_identity_recall():
    """beta_i = 1, q_i = k_i, |k_i| = 1: S_i^T k_i = S~^T k + u (k.k) = v_i, so o_i = v_i exactly
    for any tree, alpha and S0."""
    rng = np.random.default_rng(13)
    for kind in ("random", "chain", "star", "skewed"):
        T = 50
        par, _, k, v, a, _, S0 = _rand_head(rng, T, kind=kind)
        r = _run(_one_head(par, k, k, v, a, np.ones(T), S0))
        np.testing.assert_allclose(r["O"][0, :, 0], v, rtol=0, atol=1e-12)


def test_orthonormal_keys():
    """k_i = distinct basis vectors: k_i.k_j = 0 (i != j) so nodes do not couple, u_i =
    beta_i (v_i - P_i S0^T k_i) and o_i = P_i S0^T q_i + sum_{j in path(i)} Gamma_ij (q_i.k_j) u_j."""
    rng = np.random.default_rng(14)
    T, d = 60, 128
    par, q, _, v, a, b, S0 = _rand_head(rng, T)
    perm = rng.permutation(d)[:T]
    k = np.eye(d)[perm]
    r = _run(_one_head(par, q, k, v, a, b, S0))
    ell = np.zeros(T)
    for i in range(T):
        ell[i] = np.log(a[i]) + (ell[par[i]] if par[i] >= 0 else 0)
    u = b[:, None] * (v - np.exp(ell)[:, None] * (k @ S0))
    np.testing.assert_allclose(r["U"][0, :, 0], u, rtol=1e-12, atol=1e-13)
    for i in range(T):
        o = np.exp(ell[i]) * S0.T @ q[i]
        for j in synth.root_path(par, i):
            o = o + np.exp(ell[i] - ell[j]) * (q[i] @ k[j]) * u[j]
        np.testing.assert_allclose(r["O"][0, i, 0], o, rtol=1e-12, atol=1e-13)


def test_path_locality():
    """o_i on the tree equals the last output of the recurrence run on the chain path(i)."""
    rng = np.random.default_rng(15)
    T = 45
    par, q, k, v, a, b, S0 = _rand_head(rng, T)
    r = _run(_one_head(par, q, k, v, a, b, S0))
    for i in rng.choice(T, 12, replace=False):
        pth = synth.root_path(par, i)
        m = len(pth)
        rc = _run(_one_head(synth.chain(m), q[pth], k[pth], v[pth], a[pth], b[pth], S0))
        np.testing.assert_allclose(r["O"][0, i, 0], rc["O"][0, -1, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(r["U"][0, i, 0], rc["U"][0, -1, 0], rtol=0, atol=1e-13)


def test_relabeling_permutes_outputs():
    """Any topological relabelling (DFS pre-order, level order) permutes outputs identically."""
    rng = np.random.default_rng(16)
    T = 70
    par, q, k, v, a, b, S0 = _rand_head(rng, T)
    r = _run(_one_head(par, q, k, v, a, b, S0))
    for order in (synth.dfs_preorder(par), synth.level_order(par)):
        p2 = synth.relabel(par, order)
        r2 = _run(_one_head(p2, q[order], k[order], v[order], a[order], b[order], S0))
        np.testing.assert_allclose(r2["O"][0, :, 0], r["O"][0, order, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(r2["U"][0, :, 0], r["U"][0, order, 0], rtol=0, atol=1e-13)


# ------------------------------------------------------------------ the closed form (library solve)
def test_closed_form_library_solve_matches_oracle():
    """(I + G) U = R solved by numpy.linalg.solve (LAPACK) and O = diag(P) Q S0 + C U reproduce the
    oracle's U and O at d = 128 on many random trees (the page asks for 1e-10)."""
    rng = np.random.default_rng(17)
    worst = 0.0
    kinds = ["random", "skewed", "chain", "star", "level"]
    for n in range(120):
        T = int(rng.integers(1, 97))
        kind = kinds[n % len(kinds)]
        kw = {"width": int(rng.integers(1, 9))} if kind == "level" else {}
        par = synth.make_tree(kind, T, rng, **kw)
        _, q, k, v, a, b, S0 = _rand_head(rng, T, parent=par)
        if n % 7 == 0:
            a = rng.uniform(0.01, 1.0, T)  # gates down to 0.01
        r = _run(_one_head(par, q, k, v, a, b, S0))
        O, U, ell = cf.closed_form(par, q, k, v, a, b, S0, solver="dense")
        worst = max(worst, np.abs(U - r["U"][0, :, 0]).max(), np.abs(O - r["O"][0, :, 0]).max())
        np.testing.assert_allclose(ell, r["ell"][0, :, 0], rtol=1e-13, atol=1e-13)
    assert worst <= 1e-10, worst


@pytest.mark.parametrize("solver", cf.SOLVERS)
def test_every_solver_matches_oracle(solver):
    """Forward substitution, 64-node blocked substitution, the finite Neumann series with
    depth terms, the squaring form and the level-synchronous solve all give the oracle's U."""
    rng = np.random.default_rng(18)
    for kind, T in (("random", 150), ("skewed", 100), ("chain", 70), ("level", 129), ("star", 65)):
        kw = {"width": 4} if kind == "level" else {}
        par = synth.make_tree(kind, T, rng, **kw)
        _, q, k, v, a, b, S0 = _rand_head(rng, T, parent=par)
        r = _run(_one_head(par, q, k, v, a, b, S0))
        O, U, _ = cf.closed_form(par, q, k, v, a, b, S0, solver=solver)
        assert np.abs(U - r["U"][0, :, 0]).max() <= 1e-10
        assert np.abs(O - r["O"][0, :, 0]).max() <= 1e-10


def test_nilpotency():
    """G^(D+1) = 0 exactly (every product of D+1 strict-ancestor steps is empty) and G^D != 0."""
    rng = np.random.default_rng(19)
    for kind, T in (("random", 120), ("skewed", 64), ("chain", 20), ("star", 30)):
        par = synth.make_tree(kind, T, rng)
        _, q, k, v, a, b, S0 = _rand_head(rng, T, parent=par)
        G, *_ = cf.build_system(par, q, k, v, a, b, S0)
        D = int(cf.depth_of(par).max())
        Gp = np.linalg.matrix_power(G, D)
        assert np.count_nonzero(Gp) > 0
        assert np.count_nonzero(Gp @ G) == 0


def test_commit_formula_matches_oracle_state():
    """S_a = P_a S0 + sum_{j in path(a)} Gamma_aj k_j u_j^T with the oracle's U equals the
    oracle's committed state (path recurrence) and its tree state at a, for every leaf."""
    rng = np.random.default_rng(20)
    T = 64
    par, q, k, v, a, b, S0 = _rand_head(rng, T, kind="skewed")
    r = _run(_one_head(par, q, k, v, a, b, S0), all_states=True)
    for leaf in synth.leaves(par):
        pth = synth.root_path(par, int(leaf))
        pa = np.full((1, T), -1, np.int32); pa[0, :len(pth)] = pth
        S, st = oracle.commit(par[None], pa, [len(pth)], k[None, :, None], v[None, :, None],
                              a[None, :, None], b[None, :, None], S0[None, None])
        assert st[0] == 0
        Sf = cf.commit_formula(par, int(leaf), k, a, r["U"][0, :, 0], S0)
        assert np.abs(Sf - S[0, 0]).max() <= 1e-10
        assert np.abs(r["S_all"][0, leaf, 0] - S[0, 0]).max() <= 1e-12


def test_commit_status_codes():
    rng = np.random.default_rng(21)
    par = np.array([-1, 0, 0, 1, 1, 2, 2], np.int32)
    T = 7
    _, q, k, v, a, b, S0 = _rand_head(rng, T, dk=8, dv=8, parent=par)
    cases = [([0, 1, 3], 3, 0), ([0, 2, 3], 3, 3), ([1, 3], 2, 1), ([0, 9], 2, 2),
             ([], 0, 0), ([0], 8, -1), ([0], -1, -1)]
    for pth, m, e in cases:
        pa = np.full((1, T), -1, np.int32); pa[0, :len(pth)] = pth
        S, st = oracle.commit(par[None], pa, [m], k[None, :, None], v[None, :, None],
                              a[None, :, None], b[None, :, None], S0[None, None])
        assert st[0] == e, (pth, m, st[0])
        if e == 0 and m == 0:
            np.testing.assert_array_equal(S[0, 0], S0)
        if e != 0:
            assert np.isnan(S).all()


# ------------------------------------------------------------------ the page's error levels
def test_fp32_closed_form_within_page_bound():
    """The fp32 closed form (log-space ratios) stays within 1e-5 of the fp64 oracle (the page's
    M1 criterion; it measured about 3e-7 at small head sizes)."""
    rng = np.random.default_rng(22)
    worst = 0.0
    for kind, T in (("random", 128), ("skewed", 64), ("topk", 16)):
        kw = {"branching": (3, 4)} if kind == "topk" else {}
        par = synth.make_tree(kind, T, rng, **kw)
        _, q, k, v, a, b, S0 = _rand_head(rng, T, parent=par)
        r = _run(_one_head(par, q, k, v, a, b, S0))
        O, U, _ = cf.closed_form(par, q.astype(np.float32), k.astype(np.float32),
                                 v.astype(np.float32), a.astype(np.float32),
                                 b.astype(np.float32), S0.astype(np.float32),
                                 solver="fwdsub", dtype=np.float32)
        worst = max(worst, np.abs(O - r["O"][0, :, 0]).max())
    assert worst <= 1e-5, worst


def test_naive_ratio_overflows_where_log_space_does_not():
    """On a 64-node chain with alpha = 0.05, fp32 ratios P_i/P_j of cumulative decays break down
    (P underflows, 0/0 and x/0 appear) while exp(l_i - l_j) stays finite and accurate."""
    rng = np.random.default_rng(23)
    T = 64
    par = synth.chain(T)
    _, q, k, v, _, b, S0 = _rand_head(rng, T, dk=32, dv=16, parent=par)
    a = np.full(T, 0.05)
    r = _run(_one_head(par, q, k, v, a, b, S0))
    f32 = dict(dtype=np.float32)
    G, C, *_ = cf.build_system(par, q, k, v, a, b, S0, naive_ratio=True, **f32)
    assert np.count_nonzero(~np.isfinite(G)) + np.count_nonzero(~np.isfinite(C)) > 0
    O, U, _ = cf.closed_form(par, q, k, v, a, b, S0, solver="fwdsub", **f32)
    assert np.isfinite(O).all()
    assert np.abs(O - r["O"][0, :, 0]).max() <= 1e-5


# ------------------------------------------------------------------ feature-drop controls
@pytest.mark.parametrize("drop", ["causal", "gamma", "strict_c", "chain"])
def test_feature_drop_controls_fail_by_far(drop):
    """Each planted mistake (causal triangle for the tree mask, decay ratios dropped, strict
    instead of inclusive C, the tree read as a chain) moves O by at least 10x the bf16 parity
    tolerance (2e-3) on the 16-node top-k tree and on a 256-node random tree, so the tolerance
    separates right from wrong."""
    for cfg in (dict(B=1, H=2, T=16, tree="topk", tree_kw={"branching": (3, 4)}),
                dict(B=1, H=2, T=256, tree="random")):
        inp = synth.make_inputs(dtype="bf16", seed=5, **cfg)
        r = oracle.gdn_tree(inp["parent"], inp["q"], inp["k"], inp["v"], inp["alpha"],
                            inp["beta"], inp["S0"])
        Om, _, _ = cf.run_batched(inp, solver="dense", drop=drop)
        err = per_head_rel_err(Om, r["O"])
        assert err >= 10 * 2e-3, (drop, cfg["T"], err)


def test_error_metric_self_check():
    x = np.zeros((1, 2, 3, 4)); y = np.ones((1, 2, 3, 4))
    assert per_head_rel_err(x, y) == 1.0
    assert state_rel_err(np.ones((1, 1, 2, 2)), np.ones((1, 1, 2, 2))) == 0.0
    assert max_rel_err([1.0, 2.0], [1.0, 4.0]) == 0.5
    y = np.array([3.0, -4.0, 1e-6])
    assert fro_rel_err(1.001 * y, y) == pytest.approx(1e-3)
    assert fro_rel_err(np.array([3.0, 0.0, 0.0]), np.array([3.0, 4.0, 0.0])) == pytest.approx(0.8)
    # the tiny third entry is below 1e-3 of the largest and is left out of the element-wise error
    assert elem_rel_err(np.array([3.003, -4.0, 5e-6]), y) == pytest.approx(1e-3)
    assert elem_rel_err(np.array([3.0, -4.4, 1e-6]), y) == pytest.approx(0.1)


# --------------------------------------------------------------------------- grouped heads, ragged
def test_ragged_prefix_equals_full_tree():
    """Parents precede children, so the first n nodes of a tree form a closed forest and their
    outputs do not depend on the later nodes: a ragged batch's sequence of n nodes must give
    the same rows as the full tree's first n rows, whatever the padding holds."""
    T = 23
    inp = synth.make_inputs(1, 2, T, tree="random", dtype="fp32", seed=71)
    full = oracle.gdn_tree(inp["parent"], inp["q"], inp["k"], inp["v"], inp["alpha"],
                           inp["beta"], inp["S0"])
    for n in (1, 9, 22):
        junk = {name: np.array(inp[name], copy=True) for name in ("q", "k", "v", "alpha", "beta")}
        par = np.array(inp["parent"], copy=True)
        par[0, n:] = -7
        for name in junk:
            junk[name][0, n:] = np.nan
        r = oracle.gdn_tree_ragged(par, [n], junk["q"], junk["k"], junk["v"], junk["alpha"],
                                   junk["beta"], inp["S0"])
        assert r["status"][0] == 0
        assert np.array_equal(r["O"][0, :n], full["O"][0, :n])
        assert np.array_equal(r["U"][0, :n], full["U"][0, :n])
        assert np.isnan(r["O"][0, n:]).all()


def test_ragged_bad_lengths():
    inp = synth.make_inputs(3, 1, 6, tree="chain", dtype="fp32", seed=72)
    r = oracle.gdn_tree_ragged(inp["parent"], [0, 7, 6], inp["q"], inp["k"], inp["v"],
                               inp["alpha"], inp["beta"], inp["S0"])
    assert r["status"].tolist() == [-1, -1, 0]
    S, st = oracle.commit_ragged(inp["parent"], [6, 0, 3], inp["path"], inp["path_len"], inp["k"],
                                 inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    # sequence 2's chain path of 6 nodes is longer than its 3-node tree
    assert st.tolist() == [0, -1, -1]


def test_grouped_heads_expand_key_heads():
    """With one q/k head serving two value heads: value heads given identical v, gates and
    state give identical outputs; each value head equals a one-to-one run with the shared key
    head's q and k; and two value heads with different inputs differ."""
    T = 12
    inp = synth.make_inputs(2, 4, T, tree="random", dtype="fp32", seed=73, HK=2)
    v, al, be, S0 = (np.array(inp[n], copy=True) for n in ("v", "alpha", "beta", "S0"))
    v[:, :, 1], al[:, :, 1], be[:, :, 1], S0[:, 1] = v[:, :, 0], al[:, :, 0], be[:, :, 0], S0[:, 0]
    r = oracle.gdn_tree_ragged(inp["parent"], None, inp["q"], inp["k"], v, al, be, S0)
    assert np.array_equal(r["O"][:, :, 0], r["O"][:, :, 1])
    assert not np.allclose(r["O"][:, :, 1], r["O"][:, :, 2])
    for j in range(4):
        kh = j // 2
        one = oracle.gdn_tree(inp["parent"], inp["q"][:, :, kh:kh + 1], inp["k"][:, :, kh:kh + 1],
                              v[:, :, j:j + 1], al[:, :, j:j + 1], be[:, :, j:j + 1], S0[:, j:j + 1])
        assert np.array_equal(r["O"][:, :, j:j + 1], one["O"])
        assert np.array_equal(r["U"][:, :, j:j + 1], one["U"])


def test_commit_ragged_matches_accepted_state():
    """The ragged, grouped commit equals the recurrence's state at the accepted node of the
    sequence's own tree (the full tree's state there, by path locality)."""
    T = 15
    lens = [15, 8]
    inp = synth.make_inputs(2, 4, T, tree="random", dtype="fp32", seed=74, HK=1, tree_len=lens)
    S, st = oracle.commit_ragged(inp["parent"], inp["tree_len"], inp["path"], inp["path_len"],
                                 inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    assert st.tolist() == [0, 0]
    for b, n in enumerate(lens):
        acc = np.array([inp["path"][b, inp["path_len"][b] - 1]], np.int32)
        sl = (slice(b, b + 1), slice(0, n))
        r = oracle.gdn_tree(inp["parent"][sl], oracle.expand_heads(inp["q"], 4)[sl],
                            oracle.expand_heads(inp["k"], 4)[sl], inp["v"][sl], inp["alpha"][sl],
                            inp["beta"][sl], inp["S0"][b:b + 1], accept=acc)
        assert state_rel_err(S[b:b + 1], r["S_accept"]) < 1e-13
