"""bench.py's host-side contract (no GPU needed)."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_records_are_tied_to_the_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123}
    (tmp_path / "bsa_fwd_traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic("w") == 123
    rec["kernel_source_sha256_16"] = "0" * 16
    (tmp_path / "bsa_fwd_traffic_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w") is None
    assert bench.load_traffic("missing") is None


def test_committed_traffic_records_are_well_formed():
    pdir = os.path.join(ROOT, "profiles")
    for name in os.listdir(pdir):
        if name.startswith("bsa_fwd_traffic_") and name.endswith(".json"):
            rec = json.load(open(os.path.join(pdir, name)))
            assert rec["hbm_bytes_per_launch"] == (rec["hbm_read_bytes_per_launch"]
                                                   + rec["hbm_write_bytes_per_launch"])
            assert len(rec["kernel_source_sha256_16"]) == 16
            assert rec["commands"]
