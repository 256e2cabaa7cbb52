"""The benchmark's command line on the CPU: it measures one GPU only and says
so (before touching a GPU) when asked for more."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_unknown_workload_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "no_such_layer"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
