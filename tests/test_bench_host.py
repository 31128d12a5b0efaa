"""Host-side logic of bench.py (CPU only): the kernel-source hash that gates
the rocprofv3 HBM-traffic figure, the lookup of that figure, and the refusal
of a run on more than one GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_drops_comments_and_blank_runs():
    src = "int a; // note\n/* block\n comment */ int b;\n\n   int  c ;  \n"
    assert bench._code_only(src) == "int a;\nint b;\nint c ;"


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    f = tmp_path / "k.hpp"
    f.write_text("int x = 1;  // first wording\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.source_hash()
    f.write_text("// a new header line\nint x = 1;  /* second wording */\n")
    assert bench.source_hash() == h0
    f.write_text("int x = 2;\n")
    assert bench.source_hash() != h0


def test_traffic_reported_only_for_the_hashed_sources(tmp_path, monkeypatch):
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps({"fa_fwd:w": {"bytes_per_launch": 123, "source_hash": bench.source_hash()},
                              "fa_fwd:old": {"bytes_per_launch": 456, "source_hash": "0" * 16}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.traffic_for("fa_fwd:w") == 123
    assert bench.traffic_for("fa_fwd:old") is None       # counters from other kernel code
    assert bench.traffic_for("fa_fwd:missing") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
