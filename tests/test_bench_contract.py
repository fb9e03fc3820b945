"""bench.py's command-line contract that holds without a GPU: more than one GPU
is refused with a message (this path has no multi-GPU mode), before any GPU
work starts."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "exactly one GPU" in (r.stdout + r.stderr)
