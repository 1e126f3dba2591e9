"""Oracle for tree-structured Gated DeltaNet verification: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg use this
package. It wraps ``gdn_tree_oracle.c``, a plain fp64 CPU implementation of the gated delta rule
run along every node's root path (the canopy project page, "The gated delta rule" and
"M1: Oracle and tree generators"), built with gcc and loaded through ctypes. It shares no code
with the HIP library and imports nothing from it.

Every function takes numpy arrays in the layouts of the C file's header and widens the
floating-point inputs exactly to fp64 (bf16 inputs must be passed as the widened values the
device reads).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_tree_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP over (batch, head))."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o",
                               tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        _lib.oracle_num_threads.restype = i
        _lib.oracle_set_threads.argtypes = [i]
        _lib.oracle_tree_check.argtypes = [i, P]
        _lib.oracle_tree_check.restype = i
        _lib.oracle_tree_structure.argtypes = [i, i, P, P, P, P]
        _lib.oracle_gdn_tree.argtypes = [i, i, i, i, i] + [P] * 12
        _lib.oracle_commit.argtypes = [i, i, i, i, i] + [P] * 10
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle runs on (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """Run later oracle calls on n OpenMP threads (timing on one core versus all of them)."""
    _load().oracle_set_threads(int(n))


def tree_structure(parent):
    """Brute-force depth [B,T], inclusive ancestor bitmask [B,T,ceil(T/32)] uint32 and tree
    status [B] (0, or 1 + the first node with parent outside -1..i-1)."""
    par = _i32(parent)
    if par.ndim == 1:
        par = par[None]
    B, T = par.shape
    W = (T + 31) // 32
    depth = np.zeros((B, T), np.int32)
    mask = np.zeros((B, T, W), np.uint32)
    status = np.zeros(B, np.int32)
    _load().oracle_tree_structure(B, T, _p(par), _p(depth), _p(mask), _p(status))
    return depth, mask, status


def gdn_tree(parent, q, k, v, alpha, beta, S0, accept=None, all_states=False):
    """Per-path recurrence. Shapes: parent [B,T], q,k [B,T,H,dk], v [B,T,H,dv], alpha,beta
    [B,T,H], S0 [B,H,dk,dv]. Returns dict with O, U [B,T,H,dv], ell [B,T,H] (fp64), and
    S_accept [B,H,dk,dv] if ``accept`` (node id per sequence, -1 for S0) is given, and S_all
    [B,T,H,dk,dv] if ``all_states``."""
    par, q, k, v = _i32(parent), _f64(q), _f64(k), _f64(v)
    alpha, beta, S0 = _f64(alpha), _f64(beta), _f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert par.shape == (B, T) and k.shape == q.shape and v.shape == (B, T, H, dv)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H) and S0.shape == (B, H, dk, dv)
    O = np.empty((B, T, H, dv))
    U = np.empty((B, T, H, dv))
    ell = np.empty((B, T, H))
    acc = None if accept is None else _i32(accept)
    S_acc = np.empty((B, H, dk, dv)) if accept is not None else None
    S_all = np.empty((B, T, H, dk, dv)) if all_states else None
    _load().oracle_gdn_tree(B, H, T, dk, dv, _p(par), _p(q), _p(k), _p(v), _p(alpha), _p(beta),
                            _p(S0), _p(O), _p(U), _p(ell), _p(acc), _p(S_acc), _p(S_all))
    out = dict(O=O, U=U, ell=ell)
    if S_acc is not None:
        out["S_accept"] = S_acc
    if S_all is not None:
        out["S_all"] = S_all
    return out


def commit(parent, path, path_len, k, v, alpha, beta, S0):
    """State after the recurrence over each sequence's accepted root path (path [B,T] root
    first, path_len [B]). Returns (S_new [B,H,dk,dv], status [B])."""
    par, path, plen = _i32(parent), _i32(path), _i32(path_len)
    k, v, alpha, beta, S0 = _f64(k), _f64(v), _f64(alpha), _f64(beta), _f64(S0)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S_new = np.empty((B, H, dk, dv))
    status = np.zeros(B, np.int32)
    _load().oracle_commit(B, H, T, dk, dv, _p(par), _p(path), _p(plen), _p(k), _p(v),
                          _p(alpha), _p(beta), _p(S0), _p(S_new), _p(status))
    return S_new, status


def expand_heads(x, HV):
    """q or k ([B,T,H,d]) as the HV value heads see them: each of the H heads serves HV // H
    consecutive value heads, so value head j reads head j // (HV // H) (the canopy page,
    "Design decisions / Memory layout": q and k have H heads, v, the gates and the state HV)."""
    H = x.shape[2]
    assert HV % H == 0 and HV >= H
    return np.repeat(np.asarray(x), HV // H, axis=2)


def gdn_tree_ragged(parent, tree_len, q, k, v, alpha, beta, S0):
    """Grouped value heads and a ragged batch ("Memory layout": the tree plus a per-sequence
    length): sequence b is the tree of its first tree_len[b] nodes, run through ``gdn_tree``
    on its own, with q and k expanded to the value heads. q, k [B,T,H,d]; v [B,T,HV,d];
    alpha, beta [B,T,HV]; S0 [B,HV,dk,dv]; tree_len [B] or None (all T). Returns O, U, ell
    (NaN past each sequence's length: padding rows have no value) and status [B]: -1 for a
    length outside 1..T, else the tree status of the sequence's own nodes."""
    par = _i32(parent)
    B, T = par.shape
    HV = np.asarray(v).shape[2]
    lens = np.full(B, T, np.int64) if tree_len is None else np.asarray(tree_len, np.int64)
    qe, ke = expand_heads(q, HV), expand_heads(k, HV)
    v, alpha, beta, S0 = np.asarray(v), np.asarray(alpha), np.asarray(beta), np.asarray(S0)
    O = np.full(v.shape, np.nan)
    U = np.full(v.shape, np.nan)
    ell = np.full(alpha.shape, np.nan)
    status = np.zeros(B, np.int32)
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= T:
            status[b] = -1
            continue
        sl = (slice(b, b + 1), slice(0, n))
        status[b] = tree_structure(par[sl])[2][0]
        if status[b]:
            continue
        r = gdn_tree(par[sl], qe[sl], ke[sl], v[sl], alpha[sl], beta[sl], S0[b:b + 1])
        O[b, :n], U[b, :n], ell[b, :n] = r["O"][0], r["U"][0], r["ell"][0]
    return dict(O=O, U=U, ell=ell, status=status)


def commit_ragged(parent, tree_len, path, path_len, k, v, alpha, beta, S0):
    """``commit`` for grouped value heads and a ragged batch: sequence b commits on the tree of
    its first tree_len[b] nodes (a path node at or past it breaks the path), k expanded to the
    value heads. Returns (S_new [B,HV,dk,dv], status [B]); status -1 also for a length outside
    1..T."""
    par, pth, plen = _i32(parent), _i32(path), _i32(path_len)
    B, T = par.shape
    HV = np.asarray(v).shape[2]
    lens = np.full(B, T, np.int64) if tree_len is None else np.asarray(tree_len, np.int64)
    ke = expand_heads(k, HV)
    v, alpha, beta, S0 = np.asarray(v), np.asarray(alpha), np.asarray(beta), np.asarray(S0)
    S_new = np.full(S0.shape, np.nan)
    status = np.zeros(B, np.int32)
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= T:
            status[b] = -1
            continue
        sl = (slice(b, b + 1), slice(0, n))
        s, st = commit(par[sl], pth[sl], plen[b:b + 1], ke[sl], v[sl], alpha[sl], beta[sl],
                       S0[b:b + 1])
        S_new[b], status[b] = s[0], st[0]
    return S_new, status
