"""Property test of the oracle (CPU only): hypothesis draws trees of 1 to 256 nodes from every
family with gates down to 0.01, and the oracle's per-path recurrence must agree with the page's
closed form solved by a library routine (numpy.linalg.solve) to 1e-10, and its commit with the
accepted node's state; the structure must match the brute-force ancestor walk. Derandomized."""
import numpy as np
import pytest

import oracle
import synth
import closed_form as cf

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402


def _one(parent, q, k, v, alpha, beta, S0):
    return dict(parent=np.asarray(parent)[None], q=q[None, :, None], k=k[None, :, None],
                v=v[None, :, None], alpha=np.asarray(alpha)[None, :, None],
                beta=np.asarray(beta)[None, :, None], S0=S0[None, None])


@settings(max_examples=30, deadline=None, derandomize=True, database=None)
@given(T=st.integers(1, 256), fam=st.sampled_from(["random", "skewed", "chain", "star", "level"]),
       low_gates=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_oracle_matches_library_closed_form(T, fam, low_gates, seed):
    rng = np.random.default_rng(seed)
    kw = {"width": 1 + seed % 8} if fam == "level" else {}
    par = synth.make_tree(fam, T, rng, **kw)
    q = rng.standard_normal((T, 128)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, 128)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, 128))
    a = rng.uniform(0.01, 1.0, T) if low_gates else np.exp(-np.logaddexp(0, rng.standard_normal(T)))
    b = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = 0.1 * rng.standard_normal((128, 128))
    d = _one(par, q, k, v, a, b, S0)
    leaf = int(rng.integers(0, T))
    r = oracle.gdn_tree(d["parent"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                        accept=[leaf])
    O, U, ell = cf.closed_form(par, q, k, v, a, b, S0, solver="dense")
    assert np.abs(U - r["U"][0, :, 0]).max() <= 1e-10
    assert np.abs(O - r["O"][0, :, 0]).max() <= 1e-10
    np.testing.assert_allclose(ell, r["ell"][0, :, 0], rtol=1e-13, atol=1e-13)
    # commit of the root path of `leaf` equals the recurrence's state at `leaf`
    path = [leaf]
    while par[path[-1]] >= 0:
        path.append(int(par[path[-1]]))
    path = path[::-1]
    pa = np.full((1, T), -1, np.int32)
    pa[0, :len(path)] = path
    S_new, st_ = oracle.commit(d["parent"], pa, np.array([len(path)], np.int32), d["k"], d["v"],
                               d["alpha"], d["beta"], d["S0"])
    assert st_.tolist() == [0]
    scale = max(np.abs(r["S_accept"][0, 0]).max(), 1e-30)
    assert np.abs(S_new[0, 0] - r["S_accept"][0, 0]).max() / scale <= 1e-12
    # structure: depth and inclusive masks by walking each node's parents
    dep, mask, stt = oracle.tree_structure(par)
    assert stt.tolist() == [0]
    for i in range(T):
        anc, j = [], i
        while j >= 0:
            anc.append(j)
            j = int(par[j])
        assert dep[0, i] == len(anc) - 1
        bits = np.zeros(mask.shape[2], np.uint32)
        for j in anc:
            bits[j >> 5] |= np.uint32(1 << (j & 31))
        assert np.array_equal(mask[0, i], bits)
