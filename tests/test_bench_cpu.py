"""Host-side parts of bench.py (no GPU): the one-GPU guard and the
cpu_baseline object's shape on the tiny workload."""
import os
import subprocess
import sys

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_object_on_the_tiny_workload():
    sys.path.insert(0, ROOT)
    import bench
    cfg = mi.WORKLOADS["tiny_fp32"]
    cb = bench.cpu_baseline(cfg, mi.logits(cfg), budget_s=1.0, min_s=0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "tiny_fp32" in cb["sample"] and "whole layer" in cb["sample"]
    cpu = cb["cpu"]
    assert cpu["threads_used"] == cb["cores"] and cpu["os_cpu_count"] == os.cpu_count()
    assert cpu["model"] and cpu["blas"]


def test_traffic_entries_are_keyed_to_all_library_sources(tmp_path):
    """The counter traffic applies only to the sources it was measured on:
    a change to any csrc file changes the hash."""
    sys.path.insert(0, ROOT)
    import bench
    for name in ("a.hip", "b.h"):
        (tmp_path / name).write_text("x")
    h0 = bench.src_hash(str(tmp_path))
    (tmp_path / "b.h").write_text("y")
    assert bench.src_hash(str(tmp_path)) != h0
    assert len(bench.src_hash()) == 16
