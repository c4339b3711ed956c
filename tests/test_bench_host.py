"""Host-side logic of bench.py (no GPU): the one-GPU guard, the roofline
objects and the check that counter-derived traffic belongs to the current
kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_object():
    r = bench.roofline("c1_linscan", 16 * 4096 * 1024, 0.128)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["alg_bytes_per_launch"] == 12 * 16 * 4096 * 1024
    assert r["achieved"] == pytest.approx(805306368 / 0.128e-3 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    a = bench.alu_roofline("c3_lstm", 1000, 4, 1.0)
    per = bench.ALU_SLOTS_PER_ELEMENT_ITER["c3_lstm"]
    assert a["bound"] == "alu" and a["achieved"] == pytest.approx(per * 4000 / 1e-3 / 1e12)


def test_every_workload_has_bytes_kernel_and_description():
    from nonlinear_rnn_solve_pararnn_amd import synth
    for name in bench.ALG_BYTES:
        assert name in bench.DOMINANT and name in bench.DESCRIBE and name in synth.WORKLOADS
    for newton, seq in bench.SEQUENTIAL_OF.items():
        assert newton in bench.ALG_BYTES and seq in bench.ALG_BYTES


def test_traffic_is_dropped_once_a_source_changes(monkeypatch):
    for name, t in bench.TRAFFIC.items():
        # the stored figure, or None if the sources changed since it was taken
        assert bench.measured_traffic(name) in (t["bytes"], None), name
        monkeypatch.setitem(bench.TRAFFIC, name, dict(t, sha256="0" * 16))
        assert bench.measured_traffic(name) is None
    assert bench.measured_traffic("x_lstm_step") is None


def test_path_override_is_restored(monkeypatch):
    """The modality sweep sets PARARNN_*_PATH around each call and puts back
    whatever the user had set (or nothing)."""
    monkeypatch.setenv("PARARNN_GRU_PATH", "chain")
    with bench._env("PARARNN_GRU_PATH", "step"):
        assert os.environ["PARARNN_GRU_PATH"] == "step"
    assert os.environ["PARARNN_GRU_PATH"] == "chain"
    with bench._env("PARARNN_GRU_PATH", None):
        assert "PARARNN_GRU_PATH" not in os.environ
    assert os.environ["PARARNN_GRU_PATH"] == "chain"
    monkeypatch.delenv("PARARNN_LSTM_PATH", raising=False)
    with bench._env("PARARNN_LSTM_PATH", "step"):
        assert os.environ["PARARNN_LSTM_PATH"] == "step"
    assert "PARARNN_LSTM_PATH" not in os.environ
