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


def test_gate_up_work_at_the_deepseek_v3_prefill_shape():
    # Every one of the 256 experts hit: W1 and W3 of each (2 * 2048 * 7168 bf16) and of the shared
    # expert, the token matrix u read once (8192 x 7168), and the 2048-wide activations of the
    # 65,536 routed slots and of the 8192 shared rows written once: 15.51 GB for 4.329 TFLOP.
    w = WORKLOADS["dsv3_prefill"]
    weights = (256 * 2 * 2048 * 7168 + 2 * 2048 * 7168) * 2
    u_once = 8192 * 7168 * 2
    acts = (8192 * 8 * 2048 + 8192 * 2048) * 2
    assert bench.gate_up_bytes(w, 256) == weights + u_once + acts == 15_510_536_192
    assert bench.gate_up_flops(w) == 4 * 7168 * (2048 * 8192 * 8 + 2048 * 8192) == 4_329_327_034_368


def test_layer_work_at_the_deepseek_v3_prefill_shape():
    # T (2 d E + 6 d F k + 6 d F_s) = 6.524 TFLOP; router matrix + bias, 257 experts' three
    # matrices, u and y, indices and gates = 22.88 GB (all 256 experts hit).
    w = WORKLOADS["dsv3_prefill"]
    assert w.flops == 8192 * (2 * 7168 * 256 + 6 * 7168 * 2048 * 8 + 6 * 7168 * 2048) == 6_524_055_322_624
    nbytes = (256 * 7168 * 2 + 4 * 256 + 256 * 3 * 7168 * 2048 * 2 + 3 * 7168 * 2048 * 2
              + 2 * 8192 * 7168 * 2 + 8 * 8192 * 8)
    assert bench.layer_bytes(w, 256) == nbytes == 22_875_735_040


def test_prefill_roofline_is_taken_against_the_mfma_peak():
    # The C3 gate/up kernel at 4.4283 ms: 977.6 TFLOP/s = 0.391 of the MFMA peak, although its
    # 279 FLOP/B lie under the 312.5 FLOP/B ridge; the HBM fraction is reported beside it.
    w = WORKLOADS["dsv3_prefill"]
    r = bench.roofline("gate_up", bench.gate_up_flops(w), bench.gate_up_bytes(w, 256), 4.4283,
                       19_222_097_902, bound="mfma")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(0.3911, abs=1e-4)
    assert r["flop_per_byte"] == pytest.approx(279.1, abs=0.1)
    assert r["hbm_frac"] == pytest.approx(15_510_536_192 / 4.4283e-3 / 8e12, abs=1e-4)
    assert r["traffic_over_alg"] == pytest.approx(1.239, abs=1e-3)


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


def test_parity_record_of_the_cpu_leg_on_oracle_outputs():
    # The bench's parity report, fed the oracle's own routing and outputs (rounded to bf16) as the
    # "GPU" result: it must pass; a planted wrong expert on a token that is not a near-tie, and a
    # planted output error of 2 % on one token, must each fail it.
    import numpy as np
    import torch

    import oracle
    from synthetic import make_inputs, to_numpy
    w = WORKLOADS["dsv3_prefill"].with_(name="small_dsv3", T=96, d=128, E=32, F=64, Fs=64)
    inp = make_inputs(w, seed=3, device="cpu")
    u, Wr = to_numpy(inp["u"]), to_numpy(inp["W_router"])
    W1, W3, W2 = (to_numpy(inp[n]) for n in ("W1", "W3", "W2"))
    shared = tuple(to_numpy(t) for t in inp["shared"])
    bias = inp["bias"].double().numpy()
    y, idx, g, ge, gg = oracle.forward(u, Wr, W1, W3, W2, w.k, bias=bias, shared=shared,
                                       score_fn=oracle.SIGMOID, n_groups=w.n_groups,
                                       topk_groups=w.topk_groups, route_scale=w.route_scale)
    ybf = torch.from_numpy(y).to(torch.bfloat16)
    yg = to_numpy(ybf)
    tok = np.arange(0, w.T, 3)
    args = (w, u, Wr, bias, (W1, W3, W2, shared), np.arange(w.E))
    rec, _, _ = bench.oracle_check(*args, yg, idx.astype(np.int64), g.astype(np.float32), tok, 2)
    assert rec["pass"] and rec["outputs_checked"] == tok.size and rec["tokens_routed"] == w.T
    assert rec["near_ties"] == int(((ge < 1e-5) | (gg < 1e-5)).sum())
    assert rec["rel_l2_max"] < 4e-3
    # a wrong expert on a token that is not a near-tie
    t = int(np.nonzero((ge >= 1e-5) & (gg >= 1e-5))[0][0])
    bad = idx.astype(np.int64).copy()
    bad[t, -1] = next(e for e in range(w.E) if e not in bad[t])
    rec, _, _ = bench.oracle_check(*args, yg, bad, g.astype(np.float32), tok, 2)
    assert not rec["pass"] and rec["set_mismatches_without_near_tie"] == 1
    # a 2 % error on one checked token's output
    y2 = y.copy()
    y2[tok[1]] *= 1.02
    rec, _, _ = bench.oracle_check(*args, to_numpy(torch.from_numpy(y2).to(torch.bfloat16)),
                                   idx.astype(np.int64), g.astype(np.float32), tok, 2)
    assert not rec["pass"] and rec["rel_l2_max"] > 1e-2
