"""The benchmark's command-line contract that needs no GPU: a request for
more than one GPU is refused with exit status 2 and a message, before any
GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], cwd=ROOT,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, (n, r.returncode, r.stderr)
        assert "supports --gpus 1 only" in r.stderr
        assert r.stdout == ""
