"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte count
the roofline divides by, and the rule that the HBM traffic figure is dropped as soon as
the kernel sources differ from the ones the counters were taken on."""
import json
import os
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused(root_dir):
    r = subprocess.run([sys.executable, os.path.join(root_dir, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_weight_workload():
    # bf16 input read once (2 B), nibbles (1/2 B) and one scale byte per 16 values
    # written once, and the 4-byte tensor scale: 4096 x 12288 -> 128,974,852 B
    assert bench.quant_bytes(4096, 12288) == 128_974_852
    # row-wise and column-wise outputs from one read
    assert bench.quant_bytes(8192, 4096, n_out=2) == 2 * 8192 * 4096 + 2 * (8192 * 4096 * 9 // 16) + 4


def test_traffic_needs_the_counted_sources(tmp_path, monkeypatch):
    rec = {"k": {"source_sha256": bench.source_hash(), "hbm_bytes_per_dispatch": 123}}
    path = tmp_path / "pmc.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PMC_FILE", str(path))
    assert bench.traffic_for("k") == 123
    assert bench.traffic_for("other_kernel") is None
    rec["k"]["source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.traffic_for("k") is None
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("k") is None
