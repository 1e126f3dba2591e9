"""Python binding of libcanopy: tree-structured verification of a Gated DeltaNet layer on
MI355X. Argument marshalling only: every step runs in the HIP kernels behind the C ABI of
``include/canopy.h``. PyTorch supplies device memory and the current stream.

Functions take and return torch tensors on the GPU:
  tree_prep(parent, alpha)                              -> (anc_mask, depth, ell, status)
  tree_verify(q, k, v, alpha, beta, S0, parent, ...)    -> (O, U, ell) [+ mask, depth, status]
  commit(S0, k, U, alpha, parent, path, path_len, ...)  -> (S_new, path_status)
  serial_verify(q, k, v, alpha, beta, S0, parent)       -> (O, U, snapshots, status)
  serial_commit(snapshots, S0, parent, path, path_len)  -> (S_new, path_status)
q, k, v are torch.bfloat16 or torch.float32 [B,T,H,128]; alpha, beta fp32 [B,T,H];
S0 fp32 [B,H,128,128]; parent int32 [B,T]; path int32 [B,T]; path_len int32 [B].

There is no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so that libcanopy binds to the HIP runtime torch uses

__all__ = ["load", "lib_path", "tree_prep", "tree_verify", "commit", "serial_verify",
           "serial_commit", "set_wait_bound", "workspace_bytes", "CanopyError", "SOLVERS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcanopy.so")
_lib = None

SOLVERS = {"auto": 0, "fwdsub": 1, "neumann": 2, "level": 3, "series": 4, "squaring": 5, "split": 6,
           "levelsync": 7}
# Solvers that keep T x T operators per (sequence, head) in a workspace (canopy_tree_verify_ws).
WORKSPACE_SOLVERS = ("series", "squaring", "split")
_FP32, _BF16 = 0, 1


class CanopyError(RuntimeError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libcanopy.so (built in-tree by ``build.build()``); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise CanopyError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m tree_speculative_verification_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    lib.canopy_version.restype = i
    lib.canopy_set_wait_bound.argtypes = [i]
    lib.canopy_set_wait_bound.restype = i
    lib.canopy_status_string.argtypes = [i]
    lib.canopy_status_string.restype = ctypes.c_char_p
    lib.canopy_tree_prep.argtypes = [P, P, P, i, i, i, P, P, P, P, u64]
    lib.canopy_tree_prep.restype = i
    lib.canopy_tree_verify.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, P, P, P, P, P, P, i, i,
                                       u64]
    lib.canopy_tree_verify.restype = i
    lib.canopy_tree_verify_ws.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, P, P, P, P, P, P, i,
                                          i, P, ctypes.c_size_t, u64]
    lib.canopy_tree_verify_ws.restype = i
    lib.canopy_tree_verify_static.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, P, P, P, P, P, P,
                                              i, i, u64]
    lib.canopy_tree_verify_static.restype = i
    lib.canopy_workspace_bytes.argtypes = [i, i, i, i]
    lib.canopy_workspace_bytes.restype = ctypes.c_size_t
    lib.canopy_commit.argtypes = [P, P, i, P, P, P, P, P, P, i, i, i, i, P, P, u64]
    lib.canopy_commit.restype = i
    lib.canopy_commit_verify.argtypes = [P, P, P, P, P, P, P, P, i, P, P, P, P, P, P, P, i, i, i, i, i,
                                         P, P, P, P, P, P, P, P, i, i, u64]
    lib.canopy_commit_verify.restype = i
    lib.canopy_serial_verify.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, P, P, P, P, u64]
    lib.canopy_serial_verify.restype = i
    lib.canopy_serial_commit.argtypes = [P, P, P, P, P, P, i, i, i, P, P, u64]
    lib.canopy_serial_commit.restype = i
    lib.canopy_commit_layers.argtypes = [i, P, P, i, P, P, P, P, P, P, i, i, i, i, P, P, u64]
    lib.canopy_commit_layers.restype = i
    lib.canopy_serial_commit_layers.argtypes = [i, P, P, P, P, P, P, i, i, i, P, P, u64]
    lib.canopy_serial_commit_layers.restype = i
    lib.canopy_hybrid_verify.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, P, P, P, P, u64]
    lib.canopy_hybrid_verify.restype = i
    lib.canopy_tree_conv.argtypes = [P, i, P, P, P, P, i, i, i, i, i, P, P, u64]
    lib.canopy_tree_conv.restype = i
    lib.canopy_conv_commit.argtypes = [P, i, P, P, P, P, P, i, i, i, i, P, P, u64]
    lib.canopy_conv_commit.restype = i
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        msg = load().canopy_status_string(st).decode()
        raise CanopyError(f"libcanopy status {st}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _req(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


D = 128  # d_k = d_v: every kernel is built for 128-wide heads


def _head_dim(d, name):
    """Every kernel reads and writes 128-wide key and value rows; any other width is refused
    before anything reaches the GPU."""
    if d != D:
        raise ValueError(f"{name} has head dimension {d}; libcanopy supports d_k = d_v = {D} only")


def _outs(out, B, T, HV, dev):
    """Preallocated (O, U, ell) for a verify: fp32 [B,T,HV,128] twice and fp32 [B,T,HV], on the
    inputs' device and contiguous; new tensors when ``out`` is None."""
    if out is None:
        return (torch.empty((B, T, HV, D), dtype=torch.float32, device=dev),
                torch.empty((B, T, HV, D), dtype=torch.float32, device=dev),
                torch.empty((B, T, HV), dtype=torch.float32, device=dev))
    if len(out) != 3:
        raise ValueError("out must be a tuple (O, U, ell)")
    O, U, ell = out
    _req(O, "out O", torch.float32, (B, T, HV, D))
    _req(U, "out U", torch.float32, (B, T, HV, D))
    _req(ell, "out ell", torch.float32, (B, T, HV))
    for name, t in (("out O", O), ("out U", U), ("out ell", ell)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the inputs on {dev}")
    return O, U, ell


def _tree_len(tree_len, B):
    return None if tree_len is None else _req(tree_len, "tree_len", torch.int32, (B,))


def _heads(q, v):
    """q/k heads H and value heads HV (v's head count); H must divide HV."""
    H, HV = q.shape[2], v.shape[2]
    if HV % H:
        raise ValueError(f"q/k heads ({H}) must divide value heads ({HV})")
    return H, HV


def _in_dtype(q):
    if q.dtype == torch.bfloat16:
        return _BF16
    if q.dtype == torch.float32:
        return _FP32
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {q.dtype}")


def set_wait_bound(sleeps: int) -> int:
    """Test hook: the bound (in sleeps) after which a wave stops waiting for another wave's
    result in later launches of this process (negative: the default); returns the previous
    bound. A wave that gives up writes NaN rows and tree status -2."""
    return int(load().canopy_set_wait_bound(int(sleeps)))


def tree_prep(parent, alpha, tree_len=None):
    """Ancestor bitmask [B,T,ceil(T/32)] (as int32 bit patterns), depth [B,T], ell [B,T,HV] and
    tree status [B], computed on the GPU. ``tree_len`` ([B] int32) gives ragged node counts;
    rows past a sequence's count are left unwritten."""
    B, T = parent.shape
    H = alpha.shape[2]
    _req(parent, "parent", torch.int32, (B, T))
    _req(alpha, "alpha", torch.float32, (B, T, H))
    tl = _tree_len(tree_len, B)
    W = (T + 31) // 32
    dev = parent.device
    mask = torch.empty((B, T, W), dtype=torch.int32, device=dev)
    depth = torch.empty((B, T), dtype=torch.int32, device=dev)
    ell = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(load().canopy_tree_prep(_ptr(parent), _ptr(tl), _ptr(alpha), B, H, T, _ptr(mask),
                                   _ptr(depth), _ptr(ell), _ptr(status), _stream()))
    return mask, depth, ell, status


def workspace_bytes(B, HV, T, solver):
    """Bytes of workspace the solver needs for this batch (0 for the fused solvers)."""
    return int(load().canopy_workspace_bytes(int(B), int(HV), int(T), SOLVERS[solver]))


def tree_verify(q, k, v, alpha, beta, S0, parent, solver="auto", waves=0, structure=False,
                out=None, tree_len=None, workspace=None):
    """Every node's output O and pseudo-value U ([B,T,HV,128] fp32) and ell ([B,T,HV] fp32).
    q and k are [B,T,H,128] with H dividing v's head count HV (value head j reads q/k head
    j // (HV // H)). ``tree_len`` ([B] int32) gives ragged node counts; rows past a sequence's
    count are left unwritten. With ``structure=True`` also returns the ancestor bitmask, depth
    and tree status. ``out`` may pass preallocated (O, U, ell). The matrix-form solvers
    ("series", "squaring", "split") run through canopy_tree_verify_ws with ``workspace`` (a
    uint8 tensor of at least ``workspace_bytes`` bytes), allocated here when not given."""
    B, T, H, d = q.shape
    _head_dim(d, "q")
    dt = _in_dtype(q)
    H, HV = _heads(q, v)
    for name, t in (("q", q), ("k", k)):
        _req(t, name, q.dtype, (B, T, H, d))
    _req(v, "v", q.dtype, (B, T, HV, d))
    _req(alpha, "alpha", torch.float32, (B, T, HV))
    _req(beta, "beta", torch.float32, (B, T, HV))
    _req(S0, "S0", torch.float32, (B, HV, d, d))
    _req(parent, "parent", torch.int32, (B, T))
    tl = _tree_len(tree_len, B)
    dev = q.device
    O, U, ell = _outs(out, B, T, HV, dev)
    mask = depth = status = None
    if structure:
        mask = torch.empty((B, T, (T + 31) // 32), dtype=torch.int32, device=dev)
        depth = torch.empty((B, T), dtype=torch.int32, device=dev)
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    if solver in WORKSPACE_SOLVERS:
        need = workspace_bytes(B, HV, T, solver)
        if workspace is None:
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        _req(workspace, "workspace", torch.uint8)
        _check(load().canopy_tree_verify_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                            _ptr(S0), _ptr(parent), _ptr(tl), B, H, HV, T, dt,
                                            _ptr(O), _ptr(U), _ptr(ell), _ptr(mask), _ptr(depth),
                                            _ptr(status), SOLVERS[solver], int(waves),
                                            _ptr(workspace), workspace.numel(), _stream()))
    else:
        _check(load().canopy_tree_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                         _ptr(S0), _ptr(parent), _ptr(tl), B, H, HV, T, dt, _ptr(O),
                                         _ptr(U), _ptr(ell), _ptr(mask), _ptr(depth), _ptr(status),
                                         SOLVERS[solver], int(waves), _stream()))
    if structure:
        return O, U, ell, mask, depth, status
    return O, U, ell


def commit(S0, k, U, alpha, parent, path, path_len, out=None, tree_len=None):
    """State after the accepted path: S_new [B,HV,128,128] fp32 (``out`` may be S0 itself for
    an in-place commit) and the path status [B]. k is [B,T,H,128] with H dividing U's head
    count HV; ``tree_len`` as in ``tree_verify``."""
    B, T, H, d = k.shape
    _head_dim(d, "k")
    dt = _in_dtype(k)
    H, HV = _heads(k, U)
    _req(S0, "S0", torch.float32, (B, HV, d, d))
    _req(k, "k", None, (B, T, H, d))
    _req(U, "U", torch.float32, (B, T, HV, d))
    _req(alpha, "alpha", torch.float32, (B, T, HV))
    _req(parent, "parent", torch.int32, (B, T))
    _req(path, "path", torch.int32, (B, T))
    _req(path_len, "path_len", torch.int32, (B,))
    tl = _tree_len(tree_len, B)
    S_new = torch.empty_like(S0) if out is None else _req(out, "out", torch.float32, (B, HV, d, d))
    status = torch.empty((B,), dtype=torch.int32, device=k.device)
    _check(load().canopy_commit(_ptr(S0), _ptr(k), dt, _ptr(U), _ptr(alpha), _ptr(parent),
                                _ptr(tl), _ptr(path), _ptr(path_len), B, H, HV, T, _ptr(S_new),
                                _ptr(status), _stream()))
    return S_new, status


def commit_verify(S0, k_prev, U_prev, alpha_prev, parent_prev, path, path_len, q, k, v, alpha, beta,
                  parent, solver="auto", waves=0, structure=False, S_out=None, out=None,
                  tree_len_prev=None, tree_len=None):
    """One decode step: ``commit`` of the previous tree's accepted path (its k_prev, U_prev,
    alpha_prev, parent_prev, path, path_len) into S0, then ``tree_verify`` of the new tree from
    the committed state. Returns (S_new, path status, O, U, ell) and, with ``structure=True``,
    also the ancestor bitmask, depth and tree status. ``S_out`` may be S0 (in place); ``out``
    may pass preallocated (O, U, ell), whose U may be U_prev when both trees have T rows."""
    B, T, H, d = q.shape
    _head_dim(d, "q")
    Tp = k_prev.shape[1]
    dt = _in_dtype(q)
    H, HV = _heads(q, v)
    for name, t in (("q", q), ("k", k)):
        _req(t, name, q.dtype, (B, T, H, d))
    _req(v, "v", q.dtype, (B, T, HV, d))
    _req(alpha, "alpha", torch.float32, (B, T, HV))
    _req(beta, "beta", torch.float32, (B, T, HV))
    _req(parent, "parent", torch.int32, (B, T))
    _req(S0, "S0", torch.float32, (B, HV, d, d))
    _req(k_prev, "k_prev", q.dtype, (B, Tp, H, d))
    _req(U_prev, "U_prev", torch.float32, (B, Tp, HV, d))
    _req(alpha_prev, "alpha_prev", torch.float32, (B, Tp, HV))
    _req(parent_prev, "parent_prev", torch.int32, (B, Tp))
    _req(path, "path", torch.int32, (B, Tp))
    _req(path_len, "path_len", torch.int32, (B,))
    tl = _tree_len(tree_len, B)
    tlp = _tree_len(tree_len_prev, B)
    dev = q.device
    S_new = torch.empty_like(S0) if S_out is None else _req(S_out, "S_out", torch.float32, (B, HV, d, d))
    pstatus = torch.empty((B,), dtype=torch.int32, device=dev)
    O, U, ell = _outs(out, B, T, HV, dev)
    mask = depth = status = None
    if structure:
        mask = torch.empty((B, T, (T + 31) // 32), dtype=torch.int32, device=dev)
        depth = torch.empty((B, T), dtype=torch.int32, device=dev)
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(load().canopy_commit_verify(_ptr(S0), _ptr(k_prev), _ptr(U_prev), _ptr(alpha_prev),
                                       _ptr(parent_prev), _ptr(tlp), _ptr(path), _ptr(path_len), Tp,
                                       _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(parent),
                                       _ptr(tl), B, H, HV, T, dt, _ptr(S_new), _ptr(pstatus), _ptr(O),
                                       _ptr(U), _ptr(ell), _ptr(mask), _ptr(depth), _ptr(status),
                                       SOLVERS[solver], int(waves), _stream()))
    if structure:
        return S_new, pstatus, O, U, ell, mask, depth, status
    return S_new, pstatus, O, U, ell


def serial_verify(q, k, v, alpha, beta, S0, parent, snapshots=None, tree_len=None):
    """The serial fork baseline: O, U [B,T,HV,128], every node's state snapshot
    [B,T,HV,128,128] and the tree status [B]. Heads and ``tree_len`` as in ``tree_verify``."""
    B, T, H, d = q.shape
    _head_dim(d, "q")
    dt = _in_dtype(q)
    H, HV = _heads(q, v)
    for name, t in (("q", q), ("k", k)):
        _req(t, name, q.dtype, (B, T, H, d))
    _req(v, "v", q.dtype, (B, T, HV, d))
    _req(alpha, "alpha", torch.float32, (B, T, HV))
    _req(beta, "beta", torch.float32, (B, T, HV))
    _req(S0, "S0", torch.float32, (B, HV, d, d))
    _req(parent, "parent", torch.int32, (B, T))
    tl = _tree_len(tree_len, B)
    dev = q.device
    O = torch.empty((B, T, HV, d), dtype=torch.float32, device=dev)
    U = torch.empty((B, T, HV, d), dtype=torch.float32, device=dev)
    if snapshots is None:
        snapshots = torch.empty((B, T, HV, d, d), dtype=torch.float32, device=dev)
    else:
        _req(snapshots, "snapshots", torch.float32, (B, T, HV, d, d))
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(load().canopy_serial_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(S0), _ptr(parent), _ptr(tl), B, H, HV, T, dt, _ptr(O),
                                       _ptr(U), _ptr(snapshots), _ptr(status), _stream()))
    return O, U, snapshots, status


def hybrid_verify(q, k, v, alpha, beta, S0, parent, snapshots=None, tree_len=None):
    """The chain-decomposed hybrid: O, U [B,T,HV,128], the snapshot buffer [B,T,HV,128,128]
    (only fork nodes' rows written) and the tree status [B]. Arguments as ``serial_verify``."""
    B, T, H, d = q.shape
    _head_dim(d, "q")
    dt = _in_dtype(q)
    H, HV = _heads(q, v)
    for name, t in (("q", q), ("k", k)):
        _req(t, name, q.dtype, (B, T, H, d))
    _req(v, "v", q.dtype, (B, T, HV, d))
    _req(alpha, "alpha", torch.float32, (B, T, HV))
    _req(beta, "beta", torch.float32, (B, T, HV))
    _req(S0, "S0", torch.float32, (B, HV, d, d))
    _req(parent, "parent", torch.int32, (B, T))
    tl = _tree_len(tree_len, B)
    dev = q.device
    O = torch.empty((B, T, HV, d), dtype=torch.float32, device=dev)
    U = torch.empty((B, T, HV, d), dtype=torch.float32, device=dev)
    if snapshots is None:
        snapshots = torch.empty((B, T, HV, d, d), dtype=torch.float32, device=dev)
    else:
        _req(snapshots, "snapshots", torch.float32, (B, T, HV, d, d))
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(load().canopy_hybrid_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(S0), _ptr(parent), _ptr(tl), B, H, HV, T, dt, _ptr(O),
                                       _ptr(U), _ptr(snapshots), _ptr(status), _stream()))
    return O, U, snapshots, status


def serial_commit(snapshots, S0, parent, path, path_len, out=None, tree_len=None):
    """Serial baseline commit: the snapshot of each sequence's accepted node becomes S_new
    (``out`` may be S0 for an in-place commit); returns (S_new, path_status)."""
    B, T, H, d, _ = snapshots.shape
    _head_dim(d, "snapshots")
    _req(snapshots, "snapshots", torch.float32, (B, T, H, d, d))
    _req(S0, "S0", torch.float32, (B, H, d, d))
    _req(parent, "parent", torch.int32, (B, T))
    _req(path, "path", torch.int32, (B, T))
    _req(path_len, "path_len", torch.int32, (B,))
    tl = _tree_len(tree_len, B)
    S_new = torch.empty_like(S0) if out is None else _req(out, "out", torch.float32, (B, H, d, d))
    status = torch.empty((B,), dtype=torch.int32, device=S0.device)
    _check(load().canopy_serial_commit(_ptr(snapshots), _ptr(S0), _ptr(parent), _ptr(tl),
                                       _ptr(path), _ptr(path_len), B, H, T, _ptr(S_new),
                                       _ptr(status), _stream()))
    return S_new, status


def tree_conv(x, w, conv_state, parent, silu=False, tree_len=None, out=None):
    """Root-path causal convolution of a draft tree: y [B,T,C] in x's dtype and the tree status
    [B]. x [B,T,C] (bf16 or fp32), w [C,K] fp32 (w[:, K-1] multiplies the node itself),
    conv_state [B,K-1,C] in x's dtype (the last committed inputs, oldest first)."""
    B, T, C = x.shape
    K = w.shape[1]
    dt = _in_dtype(x)
    _req(x, "x", None, (B, T, C))
    _req(w, "w", torch.float32, (C, K))
    _req(conv_state, "conv_state", x.dtype, (B, K - 1, C))
    _req(parent, "parent", torch.int32, (B, T))
    tl = _tree_len(tree_len, B)
    y = torch.empty_like(x) if out is None else _req(out, "out", x.dtype, (B, T, C))
    status = torch.empty((B,), dtype=torch.int32, device=x.device)
    _check(load().canopy_tree_conv(_ptr(x), dt, _ptr(w), _ptr(conv_state), _ptr(parent), _ptr(tl),
                                   B, T, C, K, int(bool(silu)), _ptr(y), _ptr(status), _stream()))
    return y, status


def conv_commit(x, conv_state, parent, path, path_len, tree_len=None, out=None):
    """The convolution state after the accepted path ([B,K-1,C], x's dtype; ``out`` may be
    conv_state itself) and the path status [B]."""
    B, T, C = x.shape
    K = conv_state.shape[1] + 1
    dt = _in_dtype(x)
    _req(x, "x", None, (B, T, C))
    _req(conv_state, "conv_state", x.dtype, (B, K - 1, C))
    _req(parent, "parent", torch.int32, (B, T))
    _req(path, "path", torch.int32, (B, T))
    _req(path_len, "path_len", torch.int32, (B,))
    tl = _tree_len(tree_len, B)
    new = torch.empty_like(conv_state) if out is None else _req(out, "out", x.dtype, (B, K - 1, C))
    status = torch.empty((B,), dtype=torch.int32, device=x.device)
    _check(load().canopy_conv_commit(_ptr(x), dt, _ptr(conv_state), _ptr(parent), _ptr(tl),
                                     _ptr(path), _ptr(path_len), B, T, C, K, _ptr(new),
                                     _ptr(status), _stream()))
    return new, status


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    return arr


def commit_layers(S0s, ks, Us, alphas, parent, path, path_len, outs=None, tree_len=None):
    """``commit`` for L layers sharing the tree and the accepted path, in one launch: lists of
    per-layer S0, k, U and alpha (``outs`` may be the S0 list for in-place commits). Returns
    (list of S_new, path status [B])."""
    L = len(S0s)
    assert len(ks) == len(Us) == len(alphas) == L
    k0 = ks[0]
    B, T, H, d = k0.shape
    _head_dim(d, "k")
    dt = _in_dtype(k0)
    H, HV = _heads(k0, Us[0])
    for l in range(L):
        _req(S0s[l], "S0", torch.float32, (B, HV, d, d))
        _req(ks[l], "k", k0.dtype, (B, T, H, d))
        _req(Us[l], "U", torch.float32, (B, T, HV, d))
        _req(alphas[l], "alpha", torch.float32, (B, T, HV))
    _req(parent, "parent", torch.int32, (B, T))
    _req(path, "path", torch.int32, (B, T))
    _req(path_len, "path_len", torch.int32, (B,))
    tl = _tree_len(tree_len, B)
    if outs is None:
        outs = [torch.empty_like(s) for s in S0s]
    for o in outs:
        _req(o, "out", torch.float32, (B, HV, d, d))
    status = torch.empty((B,), dtype=torch.int32, device=k0.device)
    _check(load().canopy_commit_layers(L, _ptr_array(S0s), _ptr_array(ks), dt, _ptr_array(Us),
                                       _ptr_array(alphas), _ptr(parent), _ptr(tl), _ptr(path),
                                       _ptr(path_len), B, H, HV, T, _ptr_array(outs), _ptr(status),
                                       _stream()))
    return outs, status


def serial_commit_layers(snapshots, S0s, parent, path, path_len, outs=None, tree_len=None):
    """``serial_commit`` for L layers in one launch; returns (list of S_new, path status)."""
    L = len(S0s)
    B, T, H, d, _ = snapshots[0].shape
    _head_dim(d, "snapshots")
    for l in range(L):
        _req(snapshots[l], "snapshots", torch.float32, (B, T, H, d, d))
        _req(S0s[l], "S0", torch.float32, (B, H, d, d))
    _req(parent, "parent", torch.int32, (B, T))
    _req(path, "path", torch.int32, (B, T))
    _req(path_len, "path_len", torch.int32, (B,))
    tl = _tree_len(tree_len, B)
    if outs is None:
        outs = [torch.empty_like(s) for s in S0s]
    for o in outs:
        _req(o, "out", torch.float32, (B, H, d, d))
    status = torch.empty((B,), dtype=torch.int32, device=parent.device)
    _check(load().canopy_serial_commit_layers(L, _ptr_array(snapshots), _ptr_array(S0s), _ptr(parent),
                                              _ptr(tl), _ptr(path), _ptr(path_len), B, H, T,
                                              _ptr_array(outs), _ptr(status), _stream()))
    return outs, status
