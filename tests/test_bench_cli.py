"""bench.py's command-line contract on the CPU: more than one GPU is
refused with a message and a nonzero exit status before any GPU is touched
(the build runs on one GPU; the PCP rank share is its own workload)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "one GPU" in json.loads(line)["error"]
