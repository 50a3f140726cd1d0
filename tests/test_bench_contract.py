"""Host-side checks of bench.py: the one-GPU refusal, the stored counters'
reading, and the CPU baseline's record (timed here on a small workload)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import configs as C  # noqa: E402


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_counter_summary_reads_per_launch_bytes():
    name = "gpt_1.3B_x16"  # the headline workload, the one whose counters are stored
    wl = C.get(name)
    elems = wl.n * wl.N
    assert os.path.exists(bench.counter_file(name))
    assert bench.read_traffic(name, elems + 1) is None  # another launch size: not this summary
    t = bench.read_traffic(name, elems)
    if t is None:
        pytest.skip("the stored counters predate the current compress source")
    # every stream once: within 2 % of the algorithmic 12.125 B per element
    assert abs(t / (bench.B_COMPRESS * elems) - 1.0) < 0.02


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("int f(int x) { return x + 1; }  // one\n")
    b.write_text("/* other words */\nint  f(int x)\n{ return x + 1; }\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a)])
    ha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(b)])
    assert bench.kernel_source_hash() == ha
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != ha


def test_cpu_baseline_record():
    from workloads import synth as S

    wl = C.get("adam_2^20_x4")
    m = S.momentum(wl, 1, "cpu")
    x, v = S.params(wl, "cpu"), S.frozen_variance(wl, "cpu")
    rec = bench.cpu_baseline(wl, m, x, v)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["unit"] == "elements/s"
    assert rec["value"] > 0
    assert f"chunk 0 ({wl.L} elements) of all {wl.n} workers" in rec["sample"]
    mt = rec["multithreaded"]
    assert mt["value"] > 0 and mt["cores"] >= 1 and mt["unit"] == "elements/s"
    assert isinstance(rec["cpu_model"], str)


def test_step_log_lines():
    """The per-step log: one record per timed step with each call's time and
    rate and the step's worker elements/s, numbered from the first timed step."""
    ms = {"compress": [2.0, 4.0], "server": [1.0, 1.0]}
    bytes_ = {"compress": 8e9, "server": 2e9}
    lines = bench.step_log_lines(ms, 6, 10 ** 9, bytes_)
    assert [r["step"] for r in lines] == [6, 7]
    assert lines[0]["compress"]["algorithmic_GBps"] == 4000.0
    assert lines[0]["compress"]["frac_of_8TBps"] == 0.5
    assert lines[1]["calls_ms"] == 5.0
    assert lines[1]["worker_elements_per_s"] == 10 ** 9 / 5e-3
    assert bench.step_log_lines({}, 1, 1, {}) == []


@pytest.mark.parametrize("flags", [["--steps", "0"], ["--warmup", "-1"]])
def test_invalid_step_counts_are_refused(flags):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and "--steps >= 1" in res.stderr
    assert res.stdout.strip() == ""
