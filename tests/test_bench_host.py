"""bench.py's host-side contract (no GPU needed): it measures one GPU, and a
request for more exits with status 2 and a message, before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr
        assert r.stdout == ""
