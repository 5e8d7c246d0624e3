"""Host-side checks of bench.py: the one-GPU contract, the roofline record and
the algorithmic byte count it divides by (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (module level imports only the standard library)
from synthetic import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_roofline_takes_the_longer_lower_bound():
    # 1 TFLOP and 1 GB in 1 ms: the MFMA bound (0.4 ms) is longer than the HBM one (0.125 ms).
    r = bench.roofline("k", 1e12, 1e9, 1.0, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(1000.0 / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert r["hbm_frac"] == pytest.approx(1000.0 / bench.PEAK_HBM_GBS, abs=1e-4)
    # 1 GFLOP and 8 GB in 2 ms: HBM bound (1 ms against 0.4 us).
    r = bench.roofline("k", 1e9, 8e9, 2.0, 123)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(0.5)
    assert r["traffic"] == 123
    assert r["ridge_flop_per_byte"] == pytest.approx(bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9),
                                                     abs=0.05)


def test_gate_up_bytes_at_the_deepseek_v3_prefill_shape():
    # Every one of the 256 experts hit: W1 and W3 of each (2 * 2048 * 7168 bf16) and of the shared
    # expert, each of the 65,536 slots' token rows and the 8192 shared rows read once, and their
    # 2048-wide activations written once.
    w = WORKLOADS["dsv3_prefill"]
    weights = (256 * 2 * 2048 * 7168 + 2 * 2048 * 7168) * 2
    rows = (8192 * 8 + 8192) * 7168 * 2
    acts = (8192 * 8 * 2048 + 8192 * 2048) * 2
    assert bench.gate_up_bytes(w, 256) == weights + rows + acts == 16_450_060_288


def test_stored_traffic_is_used_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"source_sha": bench.kernel_source_hash(), "hbm_bytes_per_launch": 42}
    (prof / "traffic_fresh.json").write_text(json.dumps(rec))
    (prof / "traffic_stale.json").write_text(json.dumps(dict(rec, source_sha="0" * 16)))
    src = tmp_path / "mixture_experts_ffn_biased_amd" / "csrc"
    src.mkdir(parents=True)
    for f in ("gemm_stream.hip", "pipeline.hpp", "common.hpp", "plan.hpp"):
        (src / f).write_bytes(open(os.path.join(ROOT, "mixture_experts_ffn_biased_amd", "csrc", f), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("fresh") == 42
    assert bench.stored_traffic("stale") is None
    assert bench.stored_traffic("missing") is None
