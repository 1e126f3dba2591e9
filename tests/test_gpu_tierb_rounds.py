"""Tier B over 100 rounds ("M5: Commit kernel and the full round"): bf16 q/k/v with the fp32
state carried from round to round at the 9B layer's shape (B=1, H=32, a 1+3+12 top-k tree per
round with fresh inputs and a random accepted root-to-leaf path). Each round runs the decode
step (canopy_commit_verify: the previous round's path committed, then the new tree verified),
the serial fork baseline on its own carried state, and the oracle on its own. The per-round
errors against the oracle (outputs and the committed state) are printed as the error growth
curve, and so is how often the argmax of a fixed random projection of each node's output
(all 32 heads, 4096 values, to 1024 logits) differs between the parallel path, the serial
baseline and the oracle. The test bounds the drift by the bf16 tolerance at every round."""
import numpy as np
import pytest

import oracle
import synth
from _common import per_head_rel_err, state_rel_err
from gpu_util import TOL, to_device

pytestmark = pytest.mark.gpu

ROUNDS, B, H, T = 100, 1, 32, 16


@pytest.fixture(scope="module")
def canopy():
    import torch
    import tree_speculative_verification_amd as tsv
    assert torch.cuda.is_available()
    tsv.load()
    return tsv


def test_hundred_rounds_bf16(canopy):
    import torch
    proj = np.random.default_rng(77).standard_normal((H * 128, 1024))
    inp0 = synth.make_inputs(B, H, T, tree="topk", tree_kw={"branching": (3, 4)}, dtype="bf16", seed=4000)
    S_par = torch.from_numpy(inp0["S0"]).cuda()
    S_ser = S_par.clone()
    S_or = inp0["S0"].astype(np.float64)
    prev = None  # the previous round's device inputs, U and path (for the fused commit)
    flips = {"par_ser": 0, "par_or": 0, "ser_or": 0}
    worst = {"O_par": 0.0, "O_ser": 0.0, "S_par": 0.0, "S_ser": 0.0}
    for r in range(ROUNDS):
        inp = synth.make_inputs(B, H, T, tree="topk", tree_kw={"branching": (3, 4)}, dtype="bf16",
                                seed=4000 + r)
        d = to_device(inp)
        # parallel decode step: commit of round r-1's path into S_par, verify of round r's tree
        if prev is None:
            zero = torch.zeros((B,), dtype=torch.int32, device="cuda")
            S_par, pst, O, U, ell = canopy.commit_verify(S_par, d["k"], torch.zeros_like(d["v"], dtype=torch.float32),
                                                         d["alpha"], d["parent"], d["path"], zero, d["q"],
                                                         d["k"], d["v"], d["alpha"], d["beta"], d["parent"])
        else:
            S_par, pst, O, U, ell = canopy.commit_verify(S_par, prev["k"], prev["U"], prev["alpha"],
                                                         prev["parent"], prev["path"], prev["path_len"],
                                                         d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                         d["parent"])
        # serial fork baseline on its own state: verify, then commit this round's path
        O_s, U_s, snaps, st_s = canopy.serial_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_ser,
                                                     d["parent"])
        S_ser, _ = canopy.serial_commit(snaps, S_ser, d["parent"], d["path"], d["path_len"])
        torch.cuda.synchronize()
        del snaps
        # the parallel state after committing round r-1's path against the oracle's state
        s_par = state_rel_err(S_par.cpu().numpy(), S_or)
        # the oracle on its own state
        ref = oracle.gdn_tree(inp["parent"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S_or)
        O_np, Os_np = O.cpu().numpy(), O_s.cpu().numpy()
        e_par = per_head_rel_err(O_np, ref["O"])
        e_ser = per_head_rel_err(Os_np, ref["O"])
        lp = O_np.reshape(T, H * 128) @ proj
        ls = Os_np.reshape(T, H * 128) @ proj
        lo = ref["O"].reshape(T, H * 128) @ proj
        ap, as_, ao = lp.argmax(1), ls.argmax(1), lo.argmax(1)
        flips["par_ser"] += int((ap != as_).sum())
        flips["par_or"] += int((ap != ao).sum())
        flips["ser_or"] += int((as_ != ao).sum())
        # commit this round's path in the oracle; the parallel path commits it next round
        S_or, st = oracle.commit(inp["parent"], inp["path"], inp["path_len"], inp["k"], inp["v"],
                                 inp["alpha"], inp["beta"], S_or)
        assert st.tolist() == [0]
        s_ser = state_rel_err(S_ser.cpu().numpy(), S_or)
        prev = dict(k=d["k"], U=U, alpha=d["alpha"], parent=d["parent"], path=d["path"],
                    path_len=d["path_len"])
        if r == ROUNDS - 1:
            # the last round's path committed into the parallel state too: the final state
            S_fin, pst = canopy.commit(S_par, d["k"], U, d["alpha"], d["parent"], d["path"], d["path_len"])
            torch.cuda.synchronize()
            s_fin = state_rel_err(S_fin.cpu().numpy(), S_or)
            print(f"[tierb] final state S_par {s_fin:.3e} S_ser {s_ser:.3e}", flush=True)
            worst["S_par"] = max(worst["S_par"], s_fin)
        worst["S_par"] = max(worst["S_par"], s_par)
        worst["O_par"] = max(worst["O_par"], e_par)
        worst["O_ser"] = max(worst["O_ser"], e_ser)
        worst["S_ser"] = max(worst["S_ser"], s_ser)
        print(f"[tierb] round {r} O_par {e_par:.3e} O_ser {e_ser:.3e} S_par {s_par:.3e} S_ser {s_ser:.3e}"
              f" flips par_ser {flips['par_ser']} par_or {flips['par_or']} ser_or {flips['ser_or']}",
              flush=True)
        assert e_par <= TOL["bf16"] and e_ser <= TOL["bf16"], (r, e_par, e_ser)
        assert s_par <= TOL["bf16"] and s_ser <= TOL["bf16"], (r, s_par, s_ser)
    print(f"[tierb] worst {worst} flips {flips} of {ROUNDS * T} nodes", flush=True)
    assert worst["S_par"] <= TOL["bf16"]
