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
