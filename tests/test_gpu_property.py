"""Property test through the C ABI: hypothesis draws trees of 1 to 256 nodes from every family,
gates down to 0.01, the input dtype, the solver, the workgroup width and the batch shape; verify
(and the commit of the drawn path) must match the oracle within the dtype's tolerance, with the
status codes and ancestor structure exact. Derandomized, so a failure names a fixed example."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close_heads, assert_close_state, oracle_commit, run_oracle, to_device

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

pytestmark = pytest.mark.gpu

FAMILIES = ["random", "skewed", "chain", "star", "level"]


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


@settings(max_examples=40, deadline=None, derandomize=True, database=None)
@given(T=st.integers(1, 256), fam=st.sampled_from(FAMILIES), dtype=st.sampled_from(["bf16", "fp32"]),
       solver=st.sampled_from(["auto", "fwdsub", "neumann", "level"]), waves=st.sampled_from([0, 1, 2, 4, 8]),
       B=st.integers(1, 2), H=st.integers(1, 3), low_gates=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_random_layer_matches_oracle(canopy, T, fam, dtype, solver, waves, B, H, low_gates, seed):
    import torch
    kw = {"width": 1 + seed % 8} if fam == "level" else {}
    inp = synth.make_inputs(B, H, T, tree=fam, dtype=dtype, seed=seed, tree_kw=kw)
    if low_gates:
        inp["alpha"] = np.random.default_rng(seed + 1).uniform(0.01, 1.0, inp["alpha"].shape).astype(np.float32)
    d = to_device(inp)
    print("[gpu] property", T, fam, dtype, solver, waves, B, H, low_gates, seed, flush=True)
    O, U, ell, mask, depth, stt = (t.cpu().numpy() for t in canopy.tree_verify(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["parent"], solver=solver,
        waves=waves, structure=True))
    ref = run_oracle(inp)
    assert stt.tolist() == [0] * B
    assert_close_heads("O", O, ref["O"], TOL[dtype])
    assert_close_heads("U", U, ref["U"], TOL[dtype])
    d_ref, m_ref, _ = oracle.tree_structure(inp["parent"])
    assert np.array_equal(depth, d_ref)
    assert np.array_equal(mask.view(np.uint32), m_ref)
    Sn, pst = canopy.commit(d["S0"], d["k"], torch.from_numpy(U).cuda(), d["alpha"], d["parent"],
                            d["path"], d["path_len"])
    torch.cuda.synchronize()
    S_ref, st_ref = oracle_commit(inp)
    assert np.array_equal(pst.cpu().numpy(), st_ref)
    assert_close_state("S_new", Sn.cpu().numpy(), S_ref, TOL[dtype])
