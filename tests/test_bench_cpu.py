"""bench.py host logic that needs no GPU: the one-GPU refusal and the counter-file check."""

from __future__ import annotations

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_counter_traffic_follows_the_source_hash(tmp_path):
    sys.path.insert(0, ROOT)
    import bench

    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    import hashlib
    rec = {"source": os.path.relpath(str(src), ROOT), "traffic_bytes_per_launch": 1234.0,
           "source_sha256": hashlib.sha256(src.read_bytes()).hexdigest()}
    f = tmp_path / "counters.json"
    f.write_text(json.dumps(rec))
    assert bench.counter_traffic(str(f)) == 1234.0
    src.write_text("// a changed kernel\n")          # counters no longer describe the source
    assert bench.counter_traffic(str(f)) is None
    assert bench.counter_traffic(str(tmp_path / "missing.json")) is None
