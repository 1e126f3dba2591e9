"""Pins of the root-path causal convolution oracle (oracle/conv.py) to a library routine and to
invariants: a chain is numpy's causal convolution over [state; inputs]; every tree node equals
that convolution run along its own root path; committing a path and convolving the next input
equals convolving the longer chain."""
import numpy as np
import pytest
from scipy.special import expit

import synth
from oracle import conv as oc


def _draw(B, T, C, K, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, C)), rng.standard_normal((C, K)),
            rng.standard_normal((B, K - 1, C)))


def _causal(seq, w):
    """numpy's causal depthwise convolution: y[t, c] = sum_j w[c, j] seq[t + j, c] over the
    len(seq) - K + 1 full windows."""
    K = w.shape[1]
    return np.stack([np.convolve(seq[:, c], w[c, ::-1], mode="valid")
                     for c in range(seq.shape[1])], axis=1)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_chain_is_numpy_causal_convolution(K):
    B, T, C = 2, 9, 5
    x, w, st = _draw(B, T, C, K, 1 + K)
    par = np.broadcast_to(synth.chain(T), (B, T))
    y, s = oc.tree_conv(par, None, x, w, st)
    assert s.tolist() == [0, 0]
    for b in range(B):
        ref = _causal(np.concatenate([st[b], x[b]]), w)
        np.testing.assert_allclose(y[b], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tree", ["random", "skewed", "topk"])
def test_tree_node_is_its_root_path_convolution(tree):
    T, C, K = 16, 4, 4
    rng = np.random.default_rng(5)
    par = synth.make_tree(tree, T, rng, branching=(3, 4))
    x, w, st = _draw(1, T, C, K, 6)
    y, s = oc.tree_conv(par[None], None, x, w, st)
    assert s[0] == 0
    for i in range(T):
        pth = synth.root_path(par, i)
        ref = _causal(np.concatenate([st[0], x[0, pth]]), w)[-1]
        np.testing.assert_allclose(y[0, i], ref, rtol=0, atol=1e-12)


def test_silu():
    T, C, K = 7, 3, 4
    x, w, st = _draw(1, T, C, K, 7)
    par = synth.binary7()[None]
    y0, _ = oc.tree_conv(par, None, x, w, st)
    y1, _ = oc.tree_conv(par, None, x, w, st, silu=True)
    np.testing.assert_allclose(y1, y0 * expit(y0), rtol=1e-14, atol=0)


def test_second_root_reads_the_state():
    """A second root (parent -1) starts from the committed state like node 0."""
    C, K = 3, 4
    x, w, st = _draw(1, 3, C, K, 8)
    par = np.array([[-1, 0, -1]])
    y, s = oc.tree_conv(par, None, x, w, st)
    assert s[0] == 0
    ref = _causal(np.concatenate([st[0], x[0, [2]]]), w)[-1]
    np.testing.assert_allclose(y[0, 2], ref, rtol=0, atol=1e-12)


def test_commit_then_convolve_equals_longer_chain():
    """Commit a path, then convolve one more input with the new state: the same as convolving
    the whole chain (old state, path, new input) at once."""
    T, C, K = 12, 4, 4
    rng = np.random.default_rng(9)
    par = synth.random_tree(T, rng)
    x, w, st = _draw(1, T, C, K, 10)
    for a in (0, 3, 11):
        pth = synth.root_path(par, a)
        path = np.full((1, T), -1)
        path[0, :len(pth)] = pth
        new, s = oc.conv_commit(par[None], None, path, [len(pth)], x, st)
        assert s[0] == 0
        nxt = rng.standard_normal((1, 1, C))
        y_next, _ = oc.tree_conv(np.array([[-1]]), None, nxt, w, new)
        whole = _causal(np.concatenate([st[0], x[0, pth], nxt[0]]), w)[-1]
        np.testing.assert_allclose(y_next[0, 0], whole, rtol=0, atol=1e-12)
    # an empty path leaves the state as it was
    new, s = oc.conv_commit(par[None], None, np.full((1, T), -1), [0], x, st)
    assert s[0] == 0 and np.array_equal(new, st)


def test_status_codes():
    C, K = 2, 4
    x, w, st = _draw(3, 5, C, K, 11)
    par = np.array([[-1, 0, 1, 2, 3], [-1, 0, 2, 1, 0], [-1, 0, 0, 1, 1]])
    y, s = oc.tree_conv(par, [5, 5, 6], x, w, st)
    assert s.tolist() == [0, 3, -1]
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all() and np.isfinite(y[0]).all()
    y, s = oc.tree_conv(par, [5, 2, 3], x, w, st)     # bad parent past the length is padding
    assert s.tolist() == [0, 0, 0] and np.isnan(y[1, 2:]).all()
    path = np.array([[0, 1, 2, -1, -1], [0, 2, -1, -1, -1], [0, 1, 3, -1, -1]])
    new, s = oc.conv_commit(par, [5, 5, 3], path, [3, 2, 3], x, st)
    # sequence 1: node 2's parent is 2 (malformed) so the link 0 -> 2 fails at position 1;
    # sequence 2: node 3 is past the 3-node tree
    assert s.tolist() == [0, 2, 3]
    new, s = oc.conv_commit(par, [5, 5, 3], path, [6, -1, 4], x, st)
    assert s.tolist() == [-1, -1, -1]
