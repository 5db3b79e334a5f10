"""Host-side checks of bench.py: the one-GPU contract and the byte and flop
formulas its roofline uses (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_expert_matrix_bytes_match_the_workload_definition():
    # one K3 expert matrix: d*f/2 code bytes + f*d/32 scale bytes = 7,798,784 B
    cfg = synth.CONFIGS[2]
    d, f = cfg.d, cfg.f
    assert d * f // 2 + d * f // 32 == 7_798_784
    # decode gate/up: 16 experts x (gate + up), x in, h (fp32) out
    assert bench.algorithmic_bytes(cfg, 1, 16, "gateup") == 16 * 2 * 7_798_784 + d * 2 + 16 * f * 4
    # decode down: 16 experts, h in, y (fp32) out
    assert bench.algorithmic_bytes(cfg, 1, 16, "down") == 16 * 7_798_784 + 16 * f * 4 + d * 4


def test_prefill_bytes_and_flops():
    cfg = synth.CONFIGS[4]
    T, P = cfg.T, cfg.T * cfg.k
    w = 896 * 2 * 7_798_784
    split_x = 2 * T * cfg.d + 2 * T * (cfg.d // 32)  # two E4M3 terms + their scales
    split_h = 2 * P * cfg.f + 2 * P * (cfg.f // 32)  # two E4M3 terms + their scales
    assert bench.algorithmic_bytes(cfg, T, 896, "gateup") == w + split_x + split_h
    # combine: the pair slots (24-bit floats) and the routing in, y (fp32) out
    assert bench.algorithmic_bytes(cfg, T, 896, "combine") == P * cfg.d * 3 + P * 8 + T * cfg.d * 4
    # router at T=4096: 2*T*E*d flops; experts: 3 matrices of 2*d*f per pair
    flops = bench.useful_flops(cfg, T)
    assert flops == pytest.approx(2.0 * P * 3 * cfg.d * cfg.f + 2.0 * T * cfg.d * cfg.E)
    assert 5.8e12 < flops < 5.9e12


def test_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    entry = {"gemv_gateup_kernel@decode_t1": {"bytes_per_launch": 123, "source_hash": "0" * 16}}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(entry))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_source_hash", lambda: "0" * 16)
    assert bench._traffic("gemv_gateup_kernel", "decode_t1") is not None
    monkeypatch.setattr(bench, "_source_hash", lambda: "1" * 16)
    assert bench._traffic("gemv_gateup_kernel", "decode_t1") is None


def test_roofline_uses_the_timed_region_kernel_time(monkeypatch):
    """The roofline divides the dominant kernel's algorithmic bytes by its
    time inside the timed region, not by the separate all-stage pass."""
    monkeypatch.setattr(bench, "_traffic", lambda kern, workload: None)
    cfg = synth.CONFIGS[4]
    res = {"stage_ms": {"gateup": 9.0, "down": 1.0, "router_logits": 0.1, "combine": 0.1},
           "dominant": {"stage": "gateup", "ms": 4.0}, "experts_touched": 896}
    r = bench.roofline_for(cfg, cfg.T, res, "prefill_t4096")
    nbytes = bench.algorithmic_bytes(cfg, cfg.T, 896, "gateup")
    assert r["kernel_ms"] == 4.0 and r["algorithmic_bytes"] == nbytes
    assert r["achieved"] == round(nbytes / 4.0e-3 / 1e9, 1)
    assert r["frac"] == round(nbytes / 4.0e-3 / 1e9 / bench.HBM_PEAK_GBS, 4)
    assert r["kernel"] == "mx_gemm_kernel<0>"
