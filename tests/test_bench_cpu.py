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


def test_stage_flops_are_charged_to_the_stage_that_runs_them():
    """With the Memory+ gate, z = x W1 runs inside the projection GEMM: the projection is
    charged x [W_q | W1] and the gate stage only (y * silu(z)) W2."""
    sys.path.insert(0, ROOT)
    import bench
    from synth import CONFIGS

    c2 = CONFIGS["memplus_16m_bf16"]
    T = c2.T
    proj, score, gate = bench.flops(c2, T)
    assert proj == 2 * 16384 * 2048 * (4 * 512 + 2048)          # 274.9 GFLOP
    assert score == 2 * 16384 * 4 * 2 * 4096 * 256               # 274.9 GFLOP: every score once
    assert gate == 2 * 16384 * 2048 * 2048                       # 137.4 GFLOP
    c1 = CONFIGS["pkm_1m_bf16"]
    assert bench.flops(c1, c1.T) == (2 * 8192 * 1024 * 4 * 512, 2 * 8192 * 4 * 2 * 1024 * 256, 0)
    # stage times measured at the 16M-key workload (ms): every matrix rate stays below the
    # 2.5 PFLOP/s bf16 peak
    r = bench.stage_rates(c2, T, {"project": 0.2375, "score": 0.5379, "gate": 0.1056, "gather": 1.407})
    for key in ("project_TFLOPs", "score_TFLOPs", "gate_TFLOPs"):
        assert 0 < r[key] < bench.BF16_PEAK_TFLOPS, (key, r[key])
    assert abs(r["project_TFLOPs"] - 1157.5) < 1 and abs(r["gate_TFLOPs"] - 1301.4) < 1
    # a stage that did not run (NaN time, no gate) reports None rather than a rate
    r1 = bench.stage_rates(c1, c1.T, {"project": 0.05, "score": 0.1, "gate": None})
    assert r1["gate_TFLOPs"] is None and r1["project_TFLOPs"] > 0
    assert bench.stage_rates(c1, c1.T, {"score": float("nan")})["score_mfma_frac"] is None


def test_environment_names_the_seed_stack_and_sources():
    """Every bench line carries its seed, torch/HIP versions, device and a digest of the library's
    sources; on a host without a GPU the device fields are None and the line still prints."""
    sys.path.insert(0, ROOT)
    import types

    import bench

    env = bench.environment(types.SimpleNamespace(seed=7))
    assert env["seed"] == 7
    assert len(env["source_sha16"]) == 16 and int(env["source_sha16"], 16) >= 0
    assert env["source_sha16"] == bench.source_digest()      # deterministic
    assert isinstance(env["torch"], str)
    import torch
    if not torch.cuda.is_available():
        assert env["device"] is None and env["arch"] is None
