"""Host logic of bench.py (no GPU): the one-GPU contract, the code hash that keeps the
committed counter summary tied to the fused kernel's source, and the work and byte
accounting the JSON line reports."""
import os
import subprocess
import sys

import pytest
import torch

import bench
from free_block_sparse_mean_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("/* the same code,\n   other comments */ int f(int x)   {\n\n return x + 1; }\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_hash(str(a)) == bench.source_hash(str(b))
    assert bench.source_hash(str(a)) != bench.source_hash(str(c))


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    import json
    summary = tmp_path / "pmc.json"
    summary.write_text(json.dumps({"fused_src_sha256_16": bench.source_hash(bench.FUSED_SRC),
                                   "hbm_bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    # a summary taken from the current fused kernel source is reported
    assert bench.traffic_from_profile() == 123.0
    changed = tmp_path / "fused.hip"
    changed.write_text(open(bench.FUSED_SRC, encoding="utf-8").read() + "\nint extra_symbol;\n")
    monkeypatch.setattr(bench, "FUSED_SRC", str(changed))
    assert bench.traffic_from_profile() is None
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.json"))
    assert bench.traffic_from_profile() is None


@pytest.mark.parametrize("name", ["c2_video_16k", "c4_stress_128k", "c5_batched_skewed_64k"])
def test_work_accounting(name):
    w = wl.CONFIGS[name]
    nb = w.N // 64
    # every tile kept: the kept-tile work is the dense-equivalent work
    assert bench.kept_flop(w, w.B * w.H * nb * nb) == pytest.approx(bench.dense_equiv_flop(w), rel=0, abs=0)
    assert bench.kept_flop(w, 1) == 4 * 64 * 64 * w.d


def test_prepass_report():
    w = wl.CONFIGS["c4_stress_128k"]
    r = bench.prepass_report(w, 0.5)
    kv = 2 * w.B * w.H * w.N * w.d * 2
    assert r["algorithmic_bytes"] == kv
    # moved: + the bf16 V^T copy + three fp32 [n_b][d] summary arrays per head
    assert r["moved_bytes"] == kv + w.B * w.H * w.N * w.d * 2 + 3 * w.B * w.H * (w.N // 64) * w.d * 4
    assert r["hbm_gbs"] == pytest.approx(kv / 0.5e-3 / 1e9)
    assert r["frac"] == pytest.approx(r["hbm_gbs"] / bench.PEAK_HBM_GBS)
    assert r["frac_moved"] == pytest.approx(r["moved_gbs"] / bench.PEAK_HBM_GBS)
    f = bench.prepass_report(wl.CONFIGS["c1_small_f32"], 0.5)
    assert f["moved_bytes"] - f["algorithmic_bytes"] == 3 * 1 * 1 * (4096 // 64) * 64 * 4   # no V^T copy


def test_row_stats():
    kept = torch.tensor([[[10, 20, 30, 40]]], dtype=torch.int32)
    r = bench.row_stats(kept)
    assert r["mean"] == 25.0 and r["min"] == 10 and r["max"] == 40
    assert r["max_over_mean"] == pytest.approx(1.6)
    assert sum(r["hist"]) == 4 and r["hist_bin"] == 8
