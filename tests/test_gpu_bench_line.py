"""bench.py end to end on the GPU: the default workload (briefly), the layer
mode and the recurrent mode each print what the one-line JSON contract asks
for, with a roofline that agrees with its own fields and, for the default
workload, the HBM counters of the committed profile and an oracle CPU
baseline.  Each run is a child process with its own time limit."""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

pytestmark = pytest.mark.gpu

CONTRACT = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config"}


def _run(args, timeout=100):
    print("bench.py", " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert lines, r.stdout[-2000:]
    return [json.loads(l) for l in lines]


def _contract(d, steps, warmup):
    assert CONTRACT <= set(d), CONTRACT - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and math.isfinite(d["value"])
    assert d["vs_baseline"] is None
    assert d["scaling"] == "weak"
    assert "workload" in d["config"]
    assert "model" not in d["config"]


def test_default_workload_line():
    (d,) = _run(["--steps", "3", "--warmup", "1", "--cpu-budget", "2"], timeout=110)
    _contract(d, 3, 1)
    w = bench.workloads.CONFIGS["scan_2p8b_t8192_bf16"]
    assert d["config"]["workload"] == w.name and d["dtype"] == w.act and d["higher_is_better"] is True
    # value is tokens per second of the whole step
    assert d["value"] == pytest.approx(w.batch * w.seqlen / (d["ms_per_step"] / 1e3), rel=2e-3)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBPS
    assert r["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(w)[1]
    assert r["achieved"] == pytest.approx(r["algorithmic_bytes_per_launch"] / (r["launch_ms"] / 1e3) / 1e9,
                                          rel=2e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=2e-3) and 0 < r["frac"] < 1
    assert r["launch_ms"] < d["ms_per_step"]
    # counters are reported only when taken on these backward sources at this interval
    if r["traffic"] is not None:
        assert r["traffic"] >= 0.5 * r["algorithmic_bytes_per_launch"]
    a = d["alu_roofline"]
    assert a["bound"] == "alu" and 0 < a["frac"] < 1
    assert a["achieved"] == pytest.approx(a["elements_per_launch"] * a["slots_per_element"] /
                                          (r["launch_ms"] / 1e3) / 1e12, rel=5e-3)
    # the step's HBM figure is the model's bytes over the step time
    assert d["hbm_GBps"] == pytest.approx(sum(bench.algorithmic_bytes(w)) / (d["ms_per_step"] / 1e3) / 1e9,
                                          rel=2e-3)
    assert d["copy_GBps"] > 1000
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["unit"] == "tokens/s"
    assert c["precision"] == "f32" and c["host_logical_cpus"] >= c["cores"] and c["cpu_model"]
    assert "channels" in c["sample"]


def test_layer_mode_line():
    (d,) = _run(["--layer", "layer_130m_bf16", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"])
    _contract(d, 3, 1)
    assert d["config"]["workload"] == "layer_130m_bf16" and d["dtype"] == "bf16"
    assert d["fwd_ms"] > 0 and d["bwd_ms"] > 0 and d["fwd_ms"] + d["bwd_ms"] <= d["ms_per_step_eager"] * 1.05
    assert 0 < d["ms_per_step"] <= d["ms_per_step_eager"] * 1.05 and d["config"]["step"] == "HIP graph replay"
    assert d["projection_flops_per_step"] == bench.layer_flops(bench.workloads.LAYER_CONFIGS["layer_130m_bf16"])
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 2500.0
    assert abs(r["achieved"] - d["projection_flops_per_step"] / (d["ms_per_step"] / 1e3) / 1e12) <= 0.01 * r["achieved"] + 0.1


def test_recurrent_mode_lines():
    lines = _run(["--recurrent", "--steps", "20", "--warmup", "5"])
    assert lines
    for d in lines:
        assert d["higher_is_better"] is False and d["value"] > 0 and d["unit"] == "us/call"
        assert "workload" in d["config"] and d["us_per_step_graph"] > 0


def test_m3_mode_line():
    """--m3: the Mamba-3 core's line, its HBM roofline consistent with its
    own fields, the matrix-core figure beside it, the oracle CPU baseline."""
    (d,) = _run(["--m3", "m3_small_bf16", "--steps", "3", "--warmup", "1", "--cpu-budget", "2"])
    _contract(d, 3, 1)
    w = bench.workloads.M3_CONFIGS["m3_small_bf16"]
    assert d["config"]["workload"] == "m3_small_bf16" and d["dtype"] == "bf16"
    assert abs(d["value"] - w.batch * w.seqlen / (d["ms_per_step"] / 1e3)) <= 1e-3 * d["value"] + 1
    assert d["fwd_ms"] > 0 and d["bwd_ms"] > 0 and d["fwd_ms"] + d["bwd_ms"] <= d["ms_per_step_eager"] * 1.05
    assert 0 < d["ms_per_step"] <= d["ms_per_step_eager"] * 1.05 and d["config"]["step"] == "HIP graph replay"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0
    assert r["algorithmic_bytes_per_launch"] == bench.m3_bytes(w)[1]
    assert abs(r["achieved"] - r["algorithmic_bytes_per_launch"] / (r["launch_ms"] / 1e3) / 1e9) <= 0.01 * r["achieved"] + 0.2
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = d["compute_roofline"]
    assert c["bound"] == "mfma" and c["algorithmic_flops_per_launch"] == bench.m3_flops(w)[1]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
