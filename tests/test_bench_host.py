"""Host logic of bench.py (CPU only): the one-GPU contract, the validity rule of
the committed HBM-traffic record, and the algorithmic FLOP counts of the
workloads (4 d per visible (query, key) pair; causal counts only j <= i)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                         env={**os.environ, **env}, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_traffic_record_used_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.traffic_for("outlier") is None                      # no record
    rec.write_text(json.dumps({"workload": "outlier", "kernel_hash": bench.kernel_hash(),
                               "bytes_per_launch": 123456789}))
    assert bench.traffic_for("outlier") == 123456789
    assert bench.traffic_for("outlier_causal") is None               # another workload
    rec.write_text(json.dumps({"workload": "outlier", "kernel_hash": "0" * 16, "bytes_per_launch": 1}))
    assert bench.traffic_for("outlier") is None                      # counters of other sources
    rec.write_text("not json")
    assert bench.traffic_for("outlier") is None


def test_kernel_hash_covers_the_fp8_attention_sources():
    for rel in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, rel)), rel
    assert any(rel.endswith("attn_fp8.hip") for rel in bench.KERNEL_SOURCES)
    assert len(bench.kernel_hash()) == 16


# Per-call FLOP totals of the dense workloads: 4 d per visible pair, N^2 pairs per
# head, or N (N + 1) / 2 when causal.
@pytest.mark.parametrize("name,flops", [
    ("tiny", 33_554_432),
    ("outlier", 2_199_023_255_552),
    ("outlier_causal", 1_099_645_845_504),
    ("ablation", 2_338_609_692_672),
    ("channel", 1_099_645_845_504),
    ("channel_norot", 1_099_645_845_504),
])
def test_workload_flop_counts(name, flops):
    assert workloads.WORKLOADS[name].flops() == flops


def test_causal_flops_count_the_diagonal_once():
    w = workloads.WORKLOADS["outlier_causal"]
    n = w.N
    pairs = sum(i + 1 for i in range(n))                             # keys 0..i for query i
    assert w.flops() == 4 * w.D * w.B * w.H * pairs
