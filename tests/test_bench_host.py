"""Host logic of bench.py (no GPU): the one-GPU guard, the traffic figures taken from the
committed counter summaries and withheld once a kernel's sources change, and the step-time
statistics."""

from __future__ import annotations

import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_traffic_follows_the_summary_while_the_hash_matches(monkeypatch):
    text = (ROOT / "profiles" / "gemm_layer4096_bf16_hbm_traffic.md").read_text()
    recorded = text.split("kernel_hash gemm_bf16:")[1].split()[0]
    monkeypatch.setattr(bench, "kernel_hash", lambda kernel="gemm_bf16": recorded)
    rows = {c: [float(x) for x in text.split(f"launch_bytes cfg{c}:")[1].splitlines()[0].split(",")]
            for c in range(4)}
    assert all(len(v) == 16 for v in rows.values())
    launches = [(0, 0), (5, 2), (15, 0)]
    want = (rows[0][0] + rows[2][5] + rows[0][15]) / 3
    got = bench.traffic_from_profiles("gemm_bf16", "layer4096_bf16", launches)
    assert got == pytest.approx(want, rel=1e-12)
    assert bench.traffic_from_profiles("gemm_bf16", "layer4096_bf16", []) is None
    assert bench.traffic_from_profiles("gemm_bf16", "no_such_workload", launches) is None


def test_traffic_is_withheld_when_the_kernel_changed(monkeypatch):
    monkeypatch.setattr(bench, "kernel_hash", lambda kernel="gemm_bf16": "0" * 16)
    assert bench.traffic_from_profiles("gemm_bf16", "layer4096_bf16", [(0, 0)]) is None
    assert bench.shampoo_traffic_from_profile("shampoo_layer4096_f32") is None


def test_shampoo_traffic_is_the_mean_per_launch(monkeypatch):
    text = (ROOT / "profiles" / "gemm_shampoo_layer4096_f32_hbm_traffic.md").read_text()
    recorded = text.split("kernel_hash gemm_f32:")[1].split()[0]
    monkeypatch.setattr(bench, "kernel_hash", lambda kernel="gemm_f32": recorded)
    line = [l for l in text.splitlines() if l.startswith("launch_bytes:")][0]
    vals = [float(x) for x in line.split(":", 1)[1].split(",")]
    assert bench.shampoo_traffic_from_profile("shampoo_layer4096_f32") == pytest.approx(
        sum(vals) / len(vals), rel=1e-12)


class _Mark:
    def __init__(self, t):
        self.t = t

    def elapsed_time(self, other):
        return other.t - self.t


def test_step_times_median_and_min():
    marks = [_Mark(t) for t in (0.0, 10.5, 21.3, 31.6, 43.0)]   # steps 10.5, 10.8, 10.3, 11.4
    st = bench.step_times_ms(marks)
    assert st["median"] == pytest.approx(10.65) and st["min"] == pytest.approx(10.3)
    assert bench.step_times_ms(marks[:1]) == {}


class _Clock:
    """Fake device clock: a step advances it by 10 ms, or by 12 ms while profiling is on."""

    def __init__(self):
        self.t = 0.0
        self.profiling = False
        self.steps = 0
        self.prof_steps = 0

    def step(self):
        self.steps += 1
        self.prof_steps += self.profiling
        self.t += 12.0 if self.profiling else 10.0

    def record(self):
        return _Mark(self.t)


def test_timed_passes_keep_instrumentation_out_of_the_timed_steps():
    c = _Clock()

    def begin():
        c.profiling = True

    def end():
        c.profiling = False
        return {"gemm_bf16": {"launches": 3}}

    mean, per_step, stats, n_prof = bench.timed_passes(c.step, 20, c.record, lambda: None, begin, end)
    assert mean == pytest.approx(10.0)                       # the profiling cost is not in it
    assert per_step == {"median": pytest.approx(10.0), "min": pytest.approx(10.0)}
    assert stats == {"gemm_bf16": {"launches": 3}} and n_prof == 5
    assert c.steps == 20 + 20 + 5 and c.prof_steps == 5      # exactly `steps` steps per timed pass
    _, _, _, n_small = bench.timed_passes(c.step, 3, c.record, lambda: None, begin, end)
    assert n_small == 3


def test_cpu_baseline_full_and_extrapolated():
    from newton_schulz_02_amd import workloads as W

    wl = W.custom("bench_host_tiny", [(8, 24), (8, 24), (8, 24), (16, 16)], seed=3)
    full = bench.cpu_baseline(wl, full=True)
    part = bench.cpu_baseline(wl, full=False)
    assert full["extrapolated"] is False and "all 4 matrices" in full["sample"]
    assert part["extrapolated"] is True and "8x24 x3" in part["sample"] and "16x16 x1" in part["sample"]
    for r in (full, part):
        assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
        assert r["cores"] >= 1 and isinstance(r["blas"], str)
    assert "layer4096_bf16" in bench.FULL_BASELINE and "many_small_512_bf16" not in bench.FULL_BASELINE
