"""Host-side logic of bench.py (no GPU): the algorithmic byte counts behind
the roofline, the refusal of more than one GPU, and the profile readers that
attach counter figures only while the kernel sources match what was
profiled."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_b1_32k_bytes_closed_form():
    # 32,768 keys x (K + V) x 8 kv heads x 128 dims x 2 bytes
    w = workloads.make_workload("b1_32k", with_kv=False)
    assert bench.attended_tokens(w) * bench.kv_bytes_per_token(w) == 32768 * 2 * 8 * 128 * 2


def test_llama8b_bytes_from_its_lengths():
    w = workloads.make_workload("llama8b", with_kv=False)
    assert bench.kv_bytes_per_token(w) == 4096
    assert bench.attended_tokens(w) == int(w.seq_lens.sum())
    assert bench.attended_tokens(w) * 4096 == 301_355_008


def test_fp8_bytes_count_the_window_only():
    w = workloads.make_workload("fp8", with_kv=False)
    assert w.sliding_window == 4096
    L = w.seq_lens.astype(np.int64)
    assert bench.attended_tokens(w) == int(np.minimum(L, 4096).sum()) < int(L.sum())
    assert bench.kv_bytes_per_token(w) == 2 * 8 * 256            # one byte per code


def test_nvfp4_bytes_count_codes_and_scales():
    w = workloads.make_workload("nvfp4", with_kv=False)
    # per token and kv head: 256 bytes of E2M1 codes + 32 E4M3 scales, for K and V
    assert bench.kv_bytes_per_token(w) == 2 * 2 * (256 + 32)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake_root(tmp_path, text):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "counters_splitk_w.txt").write_text(text)
    (tmp_path / "profiles" / "traffic_splitk_w.txt").write_text(text)
    return str(tmp_path)


COUNTERS = """# comment: source_hash: ignored
valu_busy_pct_of_simd_cycles: 39.6
mfma_busy_pct_of_simd_cycles: 11.6
valu_insts_per_wave_tile: 318
mfma_insts_per_wave_tile: 24.0  (the tile loop issues 24)
wave_cycles_issuing_pct: 45.8
wave_cycles_waiting_any_pct: 36.0
lds_bank_conflict_cycles_pct_of_cu_cycles: 4.3
bytes_per_launch: 12345
source_hash: {h}
"""


def test_profile_readers_follow_the_source_hash(tmp_path, monkeypatch):
    root = _fake_root(tmp_path, COUNTERS.format(h="abc"))
    monkeypatch.setattr(bench, "ROOT", root)
    monkeypatch.setattr(bench, "source_hash", lambda: "abc")
    rec = bench.counters_record("w")
    assert rec["valu_busy_pct_of_simd_cycles"] == 39.6 and rec["valu_insts_per_wave_tile"] == 318
    assert bench.traffic_record("w", "splitk") == 12345.0
    monkeypatch.setattr(bench, "source_hash", lambda: "changed")
    assert bench.counters_record("w") is None
    assert bench.traffic_record("w", "splitk") is None
    assert bench.counters_record("missing") is None
