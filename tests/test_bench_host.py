"""Host-side logic of bench.py (no GPU): the committed rocprofv3 summaries are
used only while the measured kernel's sources still hash to the recorded
value, and --gpus N > 1 is refused."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

PROFILES = ["gate_up_gemm_traffic.md", "gate_up_gemm_counters.md"]


@pytest.mark.parametrize("name", PROFILES)
def test_recorded_profile_follows_source_hash(name, monkeypatch):
    """A committed summary is used exactly while the sources it was measured
    on hash to the recorded value (otherwise bench.py reports null)."""
    d = bench.profile_data(name)
    assert d is not None and len(d["sources_sha256_16"]) == 16 and d["sources"]
    monkeypatch.setattr(bench, "traffic_source_hash", lambda files: d["sources_sha256_16"])
    assert bench.recorded_profile(name) == d


def test_recorded_profile_rejects_changed_sources(monkeypatch):
    monkeypatch.setattr(bench, "traffic_source_hash", lambda files: "0" * 16)
    for name in PROFILES:
        assert bench.recorded_profile(name) is None


def test_recorded_profile_missing_file():
    assert bench.recorded_profile("no_such_summary.md") is None


def test_traffic_figures_are_consistent():
    d = bench.profile_data("gate_up_gemm_traffic.md")
    # scaled counters -> bytes, and the algorithmic bytes of the fused launch
    # (the scales: 256 MiB of the calibration copy over what the counters read for it)
    fetched = d["fetch_kib"] * (262144.0 / d["copy_fetch_kib"]) * 1024
    written = d["write_kib"] * (262144.0 / d["copy_write_kib"]) * 1024
    assert abs(fetched + written - d["traffic_bytes"]) <= 1e-6 * d["traffic_bytes"]
    M, K, N2 = d["shape_mkn"]
    assert d["algorithmic_bytes"] == (M * K + N2 * K + M * N2 // 2) * 2


def test_counted_mfma_work_equals_algorithmic():
    d = bench.profile_data("gate_up_gemm_counters.md")
    assert d["mfma_flop_counted"] == 2 * 4096 * 8192 * 28672
    assert 0.0 < d["mfma_util"] <= 1.0


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_decode_entry_takes_the_fastest_issue_mode():
    # 100 MB in 20 us (graph layers) = 5 TB/s; 1 GFLOP in the same time
    e = bench._decode_entry(0.030, 0.025, 0.020, 100e6, 1e9)
    assert e["issue"] == "graph_layers" and e["ms"] == 0.020
    assert abs(e["GB/s"] - 5000.0) < 1e-6 and abs(e["TFLOP/s"] - 50.0) < 1e-9
    assert abs(e["hbm_frac"] - 5000.0 / bench.PEAK_HBM_GBPS) < 1e-12
    e = bench._decode_entry(0.010, 0.025, 0.020, 100e6, 1e9)
    assert e["issue"] == "eager" and e["eager_ms"] == 0.010 and e["graph_layers_ms"] == 0.020
