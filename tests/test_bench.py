"""The bench contract on the CPU: one GPU only, the algorithmic byte and
pair counts of the named workloads, and measured traffic tied to the
kernel sources it was taken for."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    # every (batch, head) is independent: one process measures one GPU
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_allowed_pairs_closed_forms():
    import bench
    from entmax_amd.workloads import WORKLOADS, make_inputs
    # causal with a 32-key window, L = 2048: sum_i min(i + 1, 32) = 32 L - 31 * 32 / 2
    assert bench.allowed_pairs_per_head(WORKLOADS["decoder"], None) == [32 * 2048 - 496] * 8
    # bidirectional, no mask: L^2 per head
    assert bench.allowed_pairs_per_head(WORKLOADS["longctx"], None) == [8192 * 8192]
    # key padding: every query row of sequence b attends its n_b valid keys
    inp = make_inputs("encoder")
    lens = inp["key_mask"].sum(dim=1).tolist()
    assert bench.allowed_pairs_per_head(WORKLOADS["encoder"], inp["key_mask"]) == [128 * int(n) for n in lens]


def test_encoder_algorithmic_bytes():
    # Q (all rows), K and V rows of valid keys, O and tau in fp32, the mask
    import bench
    from entmax_amd.workloads import WORKLOADS, make_inputs
    inp = make_inputs("encoder")
    km = inp["key_mask"]
    B, H, L, d = 32, 12, 128, 64
    expect = B * H * L * d * 2 + 2 * int(km.sum()) * H * d * 2 + B * H * L * d * 4 + B * H * L * 4 + B * L
    assert bench.algorithmic_bytes(WORKLOADS["encoder"], km) == expect


def test_traffic_is_tied_to_the_kernel_sources(monkeypatch):
    # counters taken for other kernel sources are never reported
    import bench
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 64)
    for name in ("encoder", "decoder", "long", "longctx"):
        assert bench.measured_traffic(name) is None
    assert bench.measured_traffic("longctx", "bwd") is None
