"""Host-side pieces of bench.py (no GPU): metric naming, the one-GPU guard,
the CPU model string and the traffic-record lookup."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_metric_is_the_long_context_forward():
    cfg = {"workload": bench.HEADLINE_WORKLOAD}
    assert bench.metric_name(cfg, False, "bf16") == bench.METRIC
    assert bench.metric_name(cfg, True, "bf16") == bench.METRIC_BWD


def test_other_workloads_name_layout_mask_grouping_and_peak():
    fp8 = {"workload": "dense_fp8", "layout": "dense", "causal": True, "window": 0,
           "heads": 32, "kv_heads": 8}
    assert bench.metric_name(fp8, False, "fp8") == \
        "dense causal GQA attn fwd TFLOP/s on 1 MI355X; % of fp8 MFMA peak"
    win = dict(fp8, workload="dense_bf16_window", window=4096)
    assert bench.metric_name(win, True, "bf16").startswith("dense windowed GQA attn bwd")
    mha = {"workload": "varlen_f32_mha", "layout": "packed varlen", "causal": False,
           "heads": 4, "kv_heads": 4}
    assert bench.metric_name(mha, False, "f32") == \
        "varlen MHA attn fwd TFLOP/s on 1 MI355X; % of f32 MFMA peak"


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_model_is_named():
    m = bench.cpu_model()
    assert isinstance(m, str) and m.strip()


def test_traffic_lookup_contract():
    assert bench.measured_traffic("no_such_workload") is None
    for which in ("forward", "backward"):
        t = bench.measured_traffic(bench.HEADLINE_WORKLOAD, which)
        assert t is None or (isinstance(t, int) and t > 0)
    # a record is used only with the kernel sources it was taken on
    assert len(bench.kernel_source_digest("forward")) == 16
    assert bench.kernel_source_digest("forward") != bench.kernel_source_digest("backward")
