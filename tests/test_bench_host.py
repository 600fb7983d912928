"""Host-side behaviour of bench.py (no GPU): the single-GPU contract and the
rule that GEMM traffic counters are reported only for the sources they were
taken on."""
import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _write_profile(root, sha):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", "gemm_traffic_toy.txt"), "w") as f:
        f.write("# comment = ignored\n"
                f"gemm_source_sha256 = {sha}\n"
                "read_bytes_per_step = 1000\n"
                "write_bytes_per_step = 24\n")


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "abc")
    assert bench.gemm_traffic("toy") is None  # no file
    _write_profile(str(tmp_path), "abc")
    t = bench.gemm_traffic("toy")
    assert t["read_bytes"] == 1000 and t["write_bytes"] == 24 and t["bytes"] == 1024
    _write_profile(str(tmp_path), "other")
    assert bench.gemm_traffic("toy") is None  # taken on other sources: null


def test_source_hash_covers_the_gemm_sources():
    h = bench.gemm_source_hash()
    assert len(h) == 64
    for name in bench.GEMM_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "mixture_experts_layer_36_amd", "csrc", name))
