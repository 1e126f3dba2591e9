"""The entry point that allocates nothing (canopy_tree_verify_static): its workspace is the
library's own device array. Called through the C ABI, twice in a row (the second call on a
smaller batch, so the array holds the first call's data), each time against
canopy_tree_verify_ws on a caller workspace (bit for bit: the same kernels) and against the
oracle; a batch whose workspace exceeds the array is refused before any launch."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_util import TOL, assert_close_heads, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


def _say(*a):
    print("[gpu]", *a, flush=True)


def _call(lib, fn, d, B, H, T, solver, O, U, L, ws=None):
    P = ctypes.c_void_p
    args = [P(d["q"].data_ptr()), P(d["k"].data_ptr()), P(d["v"].data_ptr()), P(d["alpha"].data_ptr()),
            P(d["beta"].data_ptr()), P(d["S0"].data_ptr()), P(d["parent"].data_ptr()), None, B, H, H, T, 1,
            P(O.data_ptr()), P(U.data_ptr()), P(L.data_ptr()), None, None, None, solver, 0]
    if ws is not None:
        args += [P(ws.data_ptr()), ws.numel()]
    args.append(None)
    return fn(*args)


def test_static_matches_workspace_entry_point(canopy):
    import torch
    lib = canopy.load()
    cases = [(1, 32, 200, "random", 6), (1, 4, 50, "skewed", 4)]  # split, then a smaller series
    for B, H, T, tree, solver in cases:
        name = {4: "series", 5: "squaring", 6: "split"}[solver]
        _say("no-alloc entry point", B, H, T, tree, name)
        inp = synth.make_inputs(B, H, T, tree=tree, dtype="bf16", seed=880 + T)
        d = to_device(inp)
        O1 = torch.full((B, T, H, 128), float("nan"), device="cuda")
        U1, O2, U2 = torch.full_like(O1, float("nan")), torch.zeros_like(O1), torch.zeros_like(O1)
        L1 = torch.empty((B, T, H), device="cuda")
        L2 = torch.empty_like(L1)
        assert _call(lib, lib.canopy_tree_verify_static, d, B, H, T, solver, O1, U1, L1) == 0
        ws = torch.empty((canopy.workspace_bytes(B, H, T, name),), dtype=torch.uint8, device="cuda")
        assert _call(lib, lib.canopy_tree_verify_ws, d, B, H, T, solver, O2, U2, L2, ws) == 0
        torch.cuda.synchronize()
        assert torch.equal(O1, O2) and torch.equal(U1, U2) and torch.equal(L1, L2)
        ref = run_oracle(inp)
        assert_close_heads("O", O1.cpu().numpy(), ref["O"], TOL["bf16"])
        assert_close_heads("U", U1.cpu().numpy(), ref["U"], TOL["bf16"])


def test_static_refuses_batches_beyond_its_array(canopy):
    """SPLIT at T = 256 needs about 2.8 MiB per (sequence, head): 32 heads exceed the 64 MiB
    array, and the call returns CANOPY_ERR_WORKSPACE without touching its arguments."""
    import torch
    lib = canopy.load()
    B, H, T = 1, 32, 256
    assert canopy.workspace_bytes(B, H, T, "split") > 64 << 20
    inp = synth.make_inputs(B, H, T, tree="random", dtype="bf16", seed=890)
    d = to_device(inp)
    O = torch.full((B, T, H, 128), 5.0, device="cuda")
    U, L = torch.full_like(O, 5.0), torch.full((B, T, H), 5.0, device="cuda")
    assert _call(lib, lib.canopy_tree_verify_static, d, B, H, T, 6, O, U, L) == 3
    torch.cuda.synchronize()
    assert bool((O == 5.0).all()) and bool((U == 5.0).all())
