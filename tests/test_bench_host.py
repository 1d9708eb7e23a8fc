"""Host-side logic of bench.py (no GPU): the roofline arithmetic, the guard
on the committed HBM-counter table, and the one-GPU contract."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_dominant_is_the_slowest_tile_kernel_and_its_rate_is_per_launch():
    steps = 4
    # name: (launches, total ms over the timed steps)
    prof = {"compact": (8, 0.05), "topk_fwd_tile": (4, 11.6), "topk_dz_tile": (8, 12.8), "dh_tile": (8, 11.2)}
    flops = {"topk_fwd_tile": 3.2e12, "topk_dz_tile": 3.2e12, "dh_tile": 3.2e12}  # per step
    dom, tflops = bench.dominant(prof, flops, steps)
    assert dom == "topk_dz_tile"
    # two launches per step: 1.6e12 flops per launch over 1.6 ms each
    assert tflops == pytest.approx(1.6e12 / 1.6e-3 / 1e12)


def test_kernel_table_shares():
    # shares of the kernel pass's own GPU time; per-step times over its steps
    t = bench.kernel_table({"a": (2, 3.0), "b": (1, 1.0)}, steps=2)
    assert t["a"] == {"launches": 2, "avg_ms": 1.5, "ms_per_step": 1.5, "share": 0.75}
    assert t["b"]["share"] == pytest.approx(0.25)


def test_linear_fit_of_peak_extra_memory():
    pts = [(4096, 1000 + 678 * 4096), (16384, 1000 + 678 * 16384), (262144, 1000 + 678 * 262144)]
    f = bench.linear_fit(pts)
    assert f["bytes_per_token"] == pytest.approx(678)
    assert f["bytes_const"] == pytest.approx(1000, abs=1e-6)
    assert f["max_rel_residual"] < 1e-12


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_traffic_is_null_for_another_workload_or_changed_sources(monkeypatch):
    assert bench.traffic_from_profiles("topk_dz_tile", "no_such_workload") is None
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert bench.traffic_from_profiles("topk_dz_tile", "head_topk_t4096") is None


def test_traffic_table_names_its_workload_and_digest():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        data = json.load(f)
    assert data["workload"] == "head_topk_t4096" and len(data["source_digest"]) == 64
    c = data["calibration"]
    assert c["fetch_factor"] > 0 and c["write_factor"] > 0
    for k, v in data["kernels"].items():
        assert v["bytes_per_launch"] == pytest.approx(
            v["fetch_kib"] * 1024 * c["fetch_factor"] + v["write_kib"] * 1024 * c["write_factor"], rel=1e-6), k


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_unknown_workloads_are_refused_before_any_gpu_work():
    for name in ("no_such_workload", "no_such_workload_vshard8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", name], capture_output=True,
                           text=True, timeout=300)
        assert r.returncode == 2 and "unknown workload" in r.stderr, (name, r.stderr[-300:])
