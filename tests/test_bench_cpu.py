"""bench.py's host-side pieces: argument contract and the recorded-traffic lookup (no GPU)."""
import json
import subprocess
import sys

import pytest

import bench


def test_multi_gpu_request_exits_with_message(repo_root):
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=repo_root, capture_output=True, text=True)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_recorded_traffic_requires_matching_kernel_sources(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256": bench.gemm_source_hash(),
           "workloads": {"mixtral": {"hbm_bytes_per_launch": 123}}}
    f = tmp_path / "traffic.md"
    f.write_text("# summary\n\n```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("mixtral") == 123
    assert bench.recorded_traffic("decode") is None
    rec["kernel_source_sha256"] = "0" * 64
    f.write_text("```json\n" + json.dumps(rec) + "\n```\n")
    assert bench.recorded_traffic("mixtral") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("mixtral") is None


def test_committed_traffic_record_parses():
    import re
    text = open(bench.TRAFFIC_FILE).read()
    rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    for w in ("mixtral", "fine_grained", "ep_share", "decode"):
        assert rec["workloads"][w]["hbm_bytes_per_launch"] > 0
    assert len(rec["kernel_source_sha256"]) == 64
