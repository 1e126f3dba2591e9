"""Helpers for GPU tests: upload synth inputs, run the oracle on the same values, compare."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from _common import elem_rel_err, fro_rel_err, per_head_rel_err, state_rel_err

TOL = {"bf16": 2e-3, "fp32": 1e-5}


def to_device(inp):
    """torch tensors on cuda:0 with exactly the values the oracle sees."""
    import torch
    dev = "cuda:0"
    out = {}
    if inp["dtype"] == "bf16":
        for n in ("q", "k", "v"):
            out[n] = torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        for n in ("q", "k", "v"):
            out[n] = torch.from_numpy(inp[n]).to(dev)
    for n in ("alpha", "beta", "S0"):
        out[n] = torch.from_numpy(inp[n]).to(dev)
    for n in ("parent", "path", "path_len"):
        out[n] = torch.from_numpy(inp[n].astype(np.int32)).to(dev)
    return out


def run_oracle(inp, accept=None, all_states=False):
    return oracle.gdn_tree(inp["parent"], inp["q"], inp["k"], inp["v"], inp["alpha"],
                           inp["beta"], inp["S0"], accept=accept, all_states=all_states)


def oracle_commit(inp, path=None, path_len=None, S0=None):
    return oracle.commit(inp["parent"], inp["path"] if path is None else path,
                         inp["path_len"] if path_len is None else path_len, inp["k"], inp["v"],
                         inp["alpha"], inp["beta"], inp["S0"] if S0 is None else S0)


def slice_inputs(inp, bsel, hsel):
    """The same layer restricted to batch rows ``bsel`` and heads ``hsel`` (every (b, h) is
    independent, so the oracle on the slice gives exactly the full run's values there)."""
    out = dict(inp)
    bsel = np.asarray(bsel)
    hsel = np.asarray(hsel)
    for n in ("q", "k", "v"):
        out[n] = inp[n][bsel][:, :, hsel]
    for n in ("alpha", "beta"):
        out[n] = inp[n][bsel][:, :, hsel]
    out["S0"] = inp["S0"][bsel][:, hsel]
    out["parent"] = inp["parent"][bsel]
    out["path"] = inp["path"][bsel]
    out["path_len"] = inp["path_len"][bsel]
    out["B"], out["H"] = len(bsel), len(hsel)
    return out


def assert_close_heads(name, x, y, tol):
    err = per_head_rel_err(x, y)
    assert np.isfinite(err) and err <= tol, f"{name}: max per-head relative error {err:.3e} > {tol:.1e}"
    return err


def assert_close_state(name, x, y, tol):
    err = state_rel_err(x, y)
    assert np.isfinite(err) and err <= tol, f"{name}: max per-head relative error {err:.3e} > {tol:.1e}"
    return err


def assert_ell(ell_gpu, ell_ref):
    ell_gpu = np.asarray(ell_gpu, np.float64)
    ell_ref = np.asarray(ell_ref, np.float64)
    bound = 1e-5 * np.maximum(1.0, np.abs(ell_ref))
    bad = np.abs(ell_gpu - ell_ref) > bound
    assert not bad.any(), f"ell differs at {np.argwhere(bad)[:5]}"


def report_metrics(config, name, x, y, state=False):
    """The parity metrics of one output against the oracle: the gated one (per-(batch, head)
    infinity-norm relative error), the relative Frobenius error and the worst element-wise
    relative error over entries above 1e-3 of the largest. Printed, and appended as a JSON line
    to the file named by CANOPY_PARITY_METRICS when that is set."""
    rec = {"config": config, "output": name,
           "inf_per_head": (state_rel_err if state else per_head_rel_err)(x, y),
           "frobenius": fro_rel_err(x, y), "elementwise_above_1e-3": elem_rel_err(x, y)}
    print("[metrics]", json.dumps(rec), flush=True)
    path = os.environ.get("CANOPY_PARITY_METRICS")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(rec) + "\n")
    return rec
