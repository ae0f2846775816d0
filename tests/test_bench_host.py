"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic bytes and
flops behind the roofline entries, and the rule that counter traffic is reported only
while the kernel sources match the ones the counters were taken on."""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_decode_kernel_roofline_counts_touched_expert_weights():
    shape = synth.WORKLOADS["decode"]
    r = bench.kernel_roofline(shape, "gateup", 0.025, 29)
    per_expert = 2 * shape.I * shape.H * 2            # gate + up rows, bf16
    assert per_expert == 3_145_728
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(29 * per_expert / 25e-6 / 1e9, abs=0.1)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)
    d = bench.kernel_roofline(shape, "down", 0.010, 29)
    assert d["per_launch"].startswith(f"{29 * shape.I * shape.H * 2} B")


def test_prefill_kernel_roofline_counts_expert_flops():
    shape = synth.WORKLOADS["prefill"]
    r = bench.kernel_roofline(shape, "gateup", 0.250, 128)
    R = shape.T * shape.k
    flops = 2.0 * R * shape.H * shape.I * 2
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert r["achieved"] == pytest.approx(flops / 250e-6 / 1e12, abs=0.01)
    assert "206.16 GFLOP" in r["per_launch"]


def test_step_roofline_prices_weights_router_and_activations():
    shape = synth.WORKLOADS["decode"]
    r = bench.step_roofline(shape, 0.040, 29)
    nbytes = 29 * 3 * shape.I * shape.H * 2 + shape.E * shape.H * 2 + 2 * shape.T * shape.H * 2
    assert nbytes == 137_256_960
    assert r["achieved"] == pytest.approx(nbytes / 40e-6 / 1e9, abs=0.1)
    p = bench.step_roofline(synth.WORKLOADS["prefill"], 0.5, 128)
    s = synth.WORKLOADS["prefill"]
    flops = 2.0 * s.T * s.k * s.H * s.I * 3 + 2.0 * s.T * s.E * s.H
    assert p["achieved"] == pytest.approx(flops / 0.5e-3 / 1e12, abs=0.01)


def test_counter_traffic_only_while_the_sources_match(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "mixture_experts_layer_route_amd", "csrc")
    dst = tmp_path / "mixture_experts_layer_route_amd" / "csrc"
    shutil.copytree(src, dst)
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"sources_sha256": bench.sources_sha256(),
           "kernels": {"gateup": {"hbm_bytes_per_launch": 123456}}}
    with open(tmp_path / "profiles" / "decode_traffic.json", "w") as f:
        json.dump(rec, f)
    got = bench.measured_traffic("decode", "gateup")
    assert got == 123456
    assert bench.measured_traffic("decode", "no_such_kernel") is None
    assert bench.measured_traffic("no_such_workload", "gateup") is None
    with open(dst / "combine.hip", "a") as f:
        f.write("\n")
    assert bench.measured_traffic("decode", "gateup") is None
