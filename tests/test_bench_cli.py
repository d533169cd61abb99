"""Host-side checks of the benchmark's command line (no GPU needed)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_stream_count_is_rejected():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--streams", "3"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "invalid choice" in r.stderr
