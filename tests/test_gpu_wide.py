"""Parity of the wave-per-sub-block kernel for 65-256 node trees at the batch sizes where the
library chooses it (at most 128 (sequence, head) pairs: 1, 2 or 4 column tiles per workgroup),
every (b, h) pair against the oracle."""
import numpy as np
import pytest

import synth
from gpu_util import TOL, assert_close_heads, assert_ell, run_oracle, to_device

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


@pytest.mark.parametrize("B,T,kind", [(1, 128, "random"), (2, 256, "random"), (1, 200, "skewed"),
                                      (2, 97, "chain"), (4, 256, "random"), (4, 130, "skewed"),
                                      (3, 65, "level")])
def test_wide_kernel_auto_dispatch(canopy, B, T, kind):
    import torch
    kw = {"width": 5} if kind == "level" else {}
    inp = synth.make_inputs(B, 32, T, tree=kind, dtype="bf16", seed=300 + T + B, tree_kw=kw)
    d = to_device(inp)
    ref = run_oracle(inp)
    for solver, waves in (("auto", 0), ("fwdsub", 1), ("fwdsub", 2)):
        _say("wide", B, T, kind, solver, waves)
        O, U, ell = canopy.tree_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                       d["parent"], solver=solver, waves=waves)
        torch.cuda.synchronize()
        O, U, ell = O.cpu().numpy(), U.cpu().numpy(), ell.cpu().numpy()
        assert_close_heads("O", O, ref["O"], TOL["bf16"])
        assert_close_heads("U", U, ref["U"], TOL["bf16"])
        assert_ell(ell, ref["ell"])
