"""Host-side checks of the benchmark's command line."""

import os
import subprocess
import sys


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's share: --gpus above 1 exits non-zero with
    a message, before any GPU work."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert p.returncode != 0
    assert "exactly one GPU" in p.stderr
    assert p.stdout.strip() == ""
