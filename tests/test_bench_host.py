"""Host-side logic of the benchmark (no GPU): the algorithmic byte and flop counts behind the
roofline fractions, checked against the workload table's figures (bytes per node and head,
per-launch totals at C1-C4); the kernel the bench names for each size; the traffic file's
digest gate; the warm/cold split of a kernel trace; the one-GPU exit."""
import csv
import json
import os

import pytest

import bench


def test_bytes_per_node_and_head():
    # bf16: q, k, v (768 B), alpha and beta (8 B), O and U (1,024 B), ell (4 B) = 1,804 B;
    # fp32 inputs: 2,572 B. Per (sequence, head) 64 KiB of S0, plus 4 B of parent per node.
    for dt, per in (("bf16", 1804), ("fp32", 2572)):
        one = bench.verify_bytes(1, 1, 1, dt)
        two = bench.verify_bytes(1, 1, 2, dt)
        assert two - one == per + 4
        assert one == 65536 + per + 4


@pytest.mark.parametrize("args,expect", [
    ((1, 2, 7, "fp32"), 167_108),              # C1: 0.167 MB
    ((1, 32, 16, "bf16"), 3_020_864),          # C2: 3.02 MB
    ((1, 32, 64, "bf16"), 5_792_000),          # C3 per sequence: 5.79 MB
    ((16, 32, 256, "bf16"), 270_024_704),      # C4: 270 MB
])
def test_verify_bytes_at_the_configs(args, expect):
    assert bench.verify_bytes(*args) == expect


def test_grouped_heads_and_ragged_bytes():
    # 16 q/k heads for 32 value heads: q and k bytes halve; a ragged batch counts real nodes
    full = bench.verify_bytes(1, 32, 16, "bf16")
    grouped = bench.verify_bytes(1, 32, 16, "bf16", HK=16)
    assert full - grouped == 16 * 16 * 2 * 128 * 2
    assert bench.verify_bytes(2, 32, 16, "bf16", nodes=20) < bench.verify_bytes(2, 32, 16, "bf16")


def test_commit_bytes_c2():
    # C2 commit with a 3-node path: 4.27 MB (S0 read and S_new written per head dominate)
    assert bench.commit_bytes(1, 32, 3) == 4_268_440


def test_fused_step_bytes_c2():
    # One-launch step at C2 with a 3-node path: the verify's 3.02 MB and the commit's 4.27 MB
    # with S0 (2.10 MB) read once for both
    assert bench.fused_step_bytes(1, 32, 16, "bf16", 3) == 3_020_864 + 4_268_440 - 2_097_152
    assert bench.fused_step_bytes(1, 32, 16, "bf16", 3) == 5_192_152


@pytest.mark.parametrize("T,solver,heads,waves,one", [
    (16, "auto", 32, 0, True), (7, "neumann", 512, 0, True), (16, "fwdsub", 32, 0, False),
    (16, "level", 32, 0, False), (17, "auto", 32, 0, True), (64, "auto", 32, 0, True),
    (64, "fwdsub", 64, 0, True), (64, "auto", 512, 0, False), (40, "auto", 64, 0, False),
    (64, "level", 32, 0, False), (64, "auto", 32, 8, False), (256, "auto", 32, 0, False),
    (64, "auto", 128, 0, True), (49, "auto", 96, 0, True), (48, "auto", 128, 0, False),
    (64, "auto", 129, 0, False)])
def test_one_launch_step_follows_the_dispatch(T, solver, heads, waves, one):
    assert bench.one_launch_step(T, solver, heads, waves) == one


def test_fused_kernel_name():
    assert bench.fused_kernel_name(16, "bf16") == "canopy::verify_small_kernel<true, 1, true, 1>"
    assert bench.fused_kernel_name(7, "fp32", 2, 8) == "canopy::verify_small_kernel<false, 8, true, 1>"
    # single-tile waves filling a pass (3 per SIMD on 1024 SIMDs) or more: two column tiles
    assert bench.fused_kernel_name(16, "bf16", 376) == "canopy::verify_small_kernel<true, 1, true, 1>"
    assert bench.fused_kernel_name(16, "bf16", 384) == "canopy::verify_small_kernel<true, 1, true, 2>"
    assert bench.fused_kernel_name(16, "bf16", 512) == "canopy::verify_small_kernel<true, 1, true, 2>"
    assert bench.fused_kernel_name(16, "fp32", 512) == "canopy::verify_small_kernel<false, 1, true, 1>"
    assert bench.fused_kernel_name(16, "bf16", 32, 16) == "canopy::verify_small_kernel<true, 1, true, 2>"
    assert bench.fused_kernel_name(64, "bf16", 32) == "canopy::verify_mid_kernel<true, 4, 1, true>"
    assert bench.fused_kernel_name(64, "bf16", 64) == "canopy::verify_mid_kernel<true, 4, 2, true>"
    assert bench.fused_kernel_name(64, "bf16", 128) == "canopy::verify_mid_kernel<true, 4, 2, true>"


def test_verify_flops_dense_tile():
    assert bench.verify_flops(1, 32, 16) == 37_748_736            # C2: 37.7 MFLOP
    assert bench.verify_flops(16, 32, 256) == 25_769_803_776      # C4: 25.8 GFLOP
    assert bench.verify_flops_ragged(32, [16, 16]) == bench.verify_flops(2, 32, 16)


@pytest.mark.parametrize("T,solver,heads,waves,dtype,kernel", [
    (16, "auto", 32, 0, "bf16", "verify_small_kernel"),
    (16, "neumann", 32, 0, "fp32", "verify_small_kernel"),
    (16, "fwdsub", 32, 0, "bf16", "verify_kernel"),
    (17, "auto", 32, 0, "bf16", "verify_mid_kernel"),
    (64, "level", 512, 0, "bf16", "verify_kernel"),
    (128, "auto", 64, 0, "bf16", "verify_wide_kernel"),
    (128, "auto", 128, 0, "bf16", "verify_wide_kernel"),
    (128, "auto", 256, 0, "bf16", "verify_kernel"),
    (128, "auto", 257, 0, "bf16", "verify_dual_kernel"),
    (256, "fwdsub", 32, 16, "bf16", "verify_dual_kernel"),
    (256, "auto", 512, 8, "bf16", "verify_kernel"),
    (100, "split", 512, 0, "bf16", "mat_apply_kernel"),
    (256, "fwdsub", 512, 2, "bf16", "verify_wide_kernel"),
    (256, "auto", 32, 0, "fp32", "verify_kernel"),
    (256, "auto", 32, 8, "bf16", "verify_kernel"),
])
def test_kernel_names_follow_the_dispatch(T, solver, heads, waves, dtype, kernel):
    assert bench.verify_kernel_name(T, solver, heads, waves, dtype) == kernel


def test_traffic_gated_by_digest(tmp_path, monkeypatch):
    entry = {"verify": {"hbm_bytes_per_launch": 123}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"kernel_digest": bench.kernel_digest(),
                                "workloads": {"topk16_b1:auto:0": entry}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("topk16_b1", "auto", 0) == 123
    assert bench.measured_traffic("topk16_b1", "auto", 8) is None
    assert bench.measured_traffic("topk16_b1", "auto", 0, "fused") is None
    path.write_text(json.dumps({"kernel_digest": "0" * 16, "workloads": {"topk16_b1:auto:0": entry}}))
    assert bench.measured_traffic("topk16_b1", "auto", 0) is None


def test_digest_follows_the_kernel_sources(tmp_path, monkeypatch):
    (tmp_path / "a.hip").write_text("x")
    (tmp_path / "api.hip").write_text("host side")
    monkeypatch.setattr(bench, "KERNEL_SOURCE_DIR", str(tmp_path))
    d0 = bench.kernel_digest()
    (tmp_path / "api.hip").write_text("host side, changed")
    assert bench.kernel_digest() == d0          # the C ABI file is not device code
    (tmp_path / "a.hip").write_text("y")
    assert bench.kernel_digest() != d0


def test_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "KERNEL_SOURCE_DIR", str(tmp_path))
    (tmp_path / "k.hip").write_text("int f(int x) { return x + 1; }\n")
    d0 = bench.kernel_digest()
    (tmp_path / "k.hip").write_text("// what f does\nint f(int x) {\n    return x + 1;  /* one */\n}\n")
    assert bench.kernel_digest() == d0
    (tmp_path / "k.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_digest() != d0


def test_protocol_summary_splits_warm_and_cold(tmp_path):
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, x>"
    other_fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<long>, x>"
    ver = "void canopy::verify_small_kernel<true, 1>(canopy::VerifyArgs)"
    rows, t = [], 0

    def add(name, dur):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": str(t), "End_Timestamp": str(t + dur)})
        t += dur + 100

    add(other_fill, 10)
    add(ver, 5000)          # after an int64 fill: warm
    for _ in range(3):
        add(ver, 3000)      # warm
    for d in (9000, 7000, 8000):
        add(fill, 50000)
        add(ver, d)         # cold
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    res = bench.protocol_summary(str(path), warmup=1)
    assert res["warm"]["verify_small_kernel"]["n"] == 4
    assert res["cold"]["verify_small_kernel"]["n"] == 2                 # first cold call dropped
    assert res["cold"]["verify_small_kernel"]["median_us"] == pytest.approx(7.5)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_method_flops_from_ancestor_pairs():
    """The method's own flops (the MFMA fraction's numerator) follow the trees' ancestor pairs:
    the 1+3+12 top-k tree has |A| = 3 * 1 + 12 * 2 = 27, so C2 is 34.7 MFLOP (the workload
    table's algorithmic figure, against 37.7 dense); C4's random trees come to about 9.3 GFLOP
    (against 25.8 dense); a chain has |A| = T (T - 1) / 2."""
    import numpy as np
    import synth
    par = synth.make_tree("topk", 16, np.random.default_rng(0), branching=(3, 4))
    assert bench.ancestor_pairs(par) == 27
    assert bench.method_flops([par], 32) == 34_701_312
    assert bench.ancestor_pairs(np.arange(-1, 9)) == 45
    assert bench.ancestor_pairs(np.arange(-1, 9), n=4) == 6
    inp = bench.build_inputs(bench.WORKLOADS["random256_b16"])
    f = bench.method_flops(inp["parent"], 32)
    assert 9.0e9 < f < 9.6e9, f
    assert f < bench.verify_flops(16, 32, 256) / 2.5
    assert bench.commit_flops(32, 3) == 32 * 2 * 128 * 128 * 3


def test_trace_summary_per_kernel(tmp_path):
    rows = [("void at::native::fill<float>(x)", 0, 1000),
            ("void canopy::verify_small_kernel<true, 1, true, 2>(canopy::VerifyArgs, canopy::PrevCommitArgs)", 0, 3000),
            ("void canopy::verify_small_kernel<true, 1, true, 2>(canopy::VerifyArgs, canopy::PrevCommitArgs)", 5000, 9000),
            ("void canopy::verify_small_kernel<true, 1, true, 2>(canopy::VerifyArgs, canopy::PrevCommitArgs)", 10000, 12500),
            ("void canopy::commit_kernel<true, 4>(canopy::CommitArgs)", 20000, 21500)]
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for n, a, b in rows:
            w.writerow({"Kernel_Name": n, "Start_Timestamp": a, "End_Timestamp": b})
    res = bench.trace_summary(str(path))
    assert set(res) == {"verify_small_kernel<true, 1, true, 2>", "commit_kernel<true, 4>"}
    v = res["verify_small_kernel<true, 1, true, 2>"]
    assert v["calls"] == 3 and v["median_us"] == 3.0 and v["min_us"] == 2.5
    assert v["average_us"] == pytest.approx(3.167, abs=1e-3)
    assert res["commit_kernel<true, 4>"]["median_us"] == 1.5
