"""Host-side pieces of bench.py (no GPU): the kernel-source hash that keys
the counter readings, the lookup that drops readings of another source, the
CPU model string, and the one-GPU refusal of --gpus N > 1."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a; // one\n\n/* two */ int b;\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h0 = bench.kernel_sha256()
    src.write_text("int a;   // changed comment\n/* other */ int b;\n")
    assert bench.kernel_sha256() == h0
    src.write_text("int a; int c;\n")
    assert bench.kernel_sha256() != h0


def test_measured_is_null_for_another_source(monkeypatch):
    monkeypatch.setattr(bench, "kernel_sha256", lambda: "0" * 64)
    assert bench.measured("glm_up", "fwd", "clock_GHz") is None
    monkeypatch.setattr(bench, "kernel_sha256", lambda: bench.MEASURED["kernel_sha256"])
    for p in ("fwd", "dgrad", "wgrad"):
        clk = bench.measured("glm_up", p, "clock_GHz")
        busy = bench.measured("glm_up", p, "mfma_busy")
        assert 0.5 < clk <= bench.NOMINAL_CLOCK_GHZ and 0.0 < busy <= 1.0
        assert bench.measured("glm_up", p, "traffic") > 0
    assert bench.measured("no_such_workload", "fwd", "traffic") is None


def test_cpu_model_is_a_name():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_reports_every_pass():
    """The oracle timing on a small workload: a rate, the thread count, the
    CPU model and per-pass GFLOP, seconds and GFLOP/s."""
    from moe_grouped_gemm_ragged_amd import synth
    wl = synth.by_name("glm_up_small")
    t = synth.make_inputs(wl, "cpu")
    cpu = bench.cpu_baseline(wl, t, synth, budget_s=0.3)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOP/s" and cpu["value"] > 0
    assert cpu["cores"] >= 1 and "cpu_model" in cpu
    assert set(cpu["per_pass"]) == {"forward", "dgrad", "wgrad"}
    for v in cpu["per_pass"].values():
        assert v["GFLOP"] > 0 and v["seconds"] >= 0
