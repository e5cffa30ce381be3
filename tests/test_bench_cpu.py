"""bench.py's host-side contract, without a GPU: it measures one GPU only and says so
when asked for more, before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)


def test_bench_help_lists_the_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--no-cpu-baseline"):
        assert opt in r.stdout
