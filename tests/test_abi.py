"""CPU checks of the boundary: the built library loads and exports every entry point that
include/canopy.h declares (no compute is called without a GPU)."""
from __future__ import annotations

import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "canopy.h")
LIB = os.path.join(ROOT, "tree_speculative_verification_amd", "libcanopy.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(canopy_[a-z_]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("canopy_tree_verify", "canopy_commit", "canopy_commit_verify", "canopy_serial_verify",
              "canopy_tree_prep", "canopy_tree_conv", "canopy_conv_commit", "canopy_status_string",
              "canopy_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "libcanopy.so is not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(lib, n), n
    lib.canopy_version.restype = ctypes.c_int
    assert lib.canopy_version() >= 100
    lib.canopy_status_string.restype = ctypes.c_char_p
    lib.canopy_status_string.argtypes = [ctypes.c_int]
    assert lib.canopy_status_string(0) == b"ok"


def test_host_checks_need_no_gpu():
    """Argument errors are found on the host before any HIP call, so they work without a GPU."""
    lib = ctypes.CDLL(LIB)
    f = lib.canopy_tree_verify
    f.restype = ctypes.c_int
    nul = ctypes.c_void_p(0)
    i = ctypes.c_int
    # q, k, v, alpha, beta, S0, parent, tree_len; B, H, HV, T, dtype; O, U, ell, mask, depth,
    # status; solver, waves, stream
    args = [nul] * 8 + [i(1), i(1), i(1), i(4), i(0)] + [nul] * 6 + [i(0), i(0), nul]
    assert f(*args) == 1
    g = lib.canopy_commit
    g.restype = ctypes.c_int
    # S0, k, dtype, U, alpha, parent, tree_len, path, path_len, B, H, HV, T, S_new, status, stream
    assert g(*([nul, nul, i(0), nul, nul, nul, nul, nul, nul, i(1), i(1), i(1), i(4), nul, nul,
                nul])) == 1
    cv = lib.canopy_commit_verify
    cv.restype = ctypes.c_int
    # S0, k_prev, U_prev, alpha_prev, parent_prev, tree_len_prev, path, path_len, T_prev; q, k,
    # v, alpha, beta, parent, tree_len; B, H, HV, T, dtype; S_new, path_status, O, U, ell, mask,
    # depth, status; solver, waves, stream
    assert cv(*([nul] * 8 + [i(4)] + [nul] * 7 + [i(1), i(1), i(1), i(4), i(0)] + [nul] * 8 +
                [i(0), i(0), nul])) == 1


def test_product_path_does_not_touch_the_oracle():
    """The package and its sources never name the oracle module."""
    pkg = os.path.join(ROOT, "tree_speculative_verification_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "liboracle" not in src, f


def test_conv_host_checks_need_no_gpu():
    """Convolution sizes are checked on the host: K outside 2..4 or C not a multiple of 8."""
    lib = ctypes.CDLL(LIB)
    f = lib.canopy_tree_conv
    f.restype = ctypes.c_int
    i = ctypes.c_int
    buf = ctypes.create_string_buffer(4096 + 16)
    p = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)  # aligned, never dereferenced
    nul = ctypes.c_void_p(0)
    # x, dtype, w, state, parent, tree_len, B, T, C, K, silu, y, status, stream
    def call(C, K, x=p):
        return f(x, i(0), p, p, p, nul, i(1), i(4), i(C), i(K), i(0), p, nul, nul)
    assert call(12, 4) == 1
    assert call(16, 5) == 1
    assert call(16, 1) == 1
    assert call(16, 4, x=nul) == 1


def test_binding_refuses_other_head_dims():
    """Every kernel is built for d_k = d_v = 128: the binding refuses any other width before a
    pointer reaches the library (checked first, so CPU tensors show it without a GPU)."""
    import pytest
    import torch
    import tree_speculative_verification_amd as canopy
    B, T, H, d = 1, 4, 2, 64
    q = torch.zeros((B, T, H, d), dtype=torch.bfloat16)
    a = torch.ones((B, T, H))
    S0 = torch.zeros((B, H, d, d))
    par = torch.tensor([[-1, 0, 0, 1]], dtype=torch.int32)
    with pytest.raises(ValueError, match="head dimension 64"):
        canopy.tree_verify(q, q, q, a, a, S0, par)
    with pytest.raises(ValueError, match="head dimension 64"):
        canopy.commit(S0, q, torch.zeros((B, T, H, d)), a, par, par, torch.ones(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="head dimension 64"):
        canopy.serial_verify(q, q, q, a, a, S0, par)
    with pytest.raises(ValueError, match="head dimension 64"):
        canopy.hybrid_verify(q, q, q, a, a, S0, par)
    with pytest.raises(ValueError, match="head dimension 64"):
        canopy.commit_verify(S0, q, torch.zeros((B, T, H, d)), a, par, par,
                             torch.ones(1, dtype=torch.int32), q, q, q, a, a, par)


def test_workspace_bytes_without_gpu():
    """The workspace size is host arithmetic: one slot per (sequence, value head) of a 64-byte
    header plus n fp32 Tp x Tp matrices (Tp = T rounded up to 16): n = 3 for the series,
    max(ceil(log2 T), 1) + 4 for the squaring form, 11 for the split design; 0 for the fused
    solvers and for sizes out of range."""
    lib = ctypes.CDLL(LIB)
    f = lib.canopy_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int] * 4
    assert f(1, 32, 16, 0) == 0 and f(1, 32, 16, 3) == 0
    assert f(2, 32, 256, 4) == 64 * (64 + 3 * 256 * 256 * 4)
    assert f(1, 1, 256, 5) == 64 + (8 + 4) * 256 * 256 * 4
    assert f(1, 1, 100, 5) == 64 + (7 + 4) * 112 * 112 * 4
    assert f(1, 1, 1, 5) == 64 + 5 * 16 * 16 * 4
    assert f(3, 2, 17, 6) == 6 * (64 + 11 * 32 * 32 * 4)
    assert f(1, 1, 257, 4) == 0 and f(0, 1, 16, 4) == 0
