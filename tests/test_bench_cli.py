"""The benchmark's command line refuses what it cannot run, before touching a
GPU: more than one GPU (the path has no multi-GPU part) and a paged cache for
a prefill workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_paged_prefill_is_refused():
    r = _run("--config", "2", "--paged")
    assert r.returncode == 2
    assert "decode workloads" in r.stderr
