"""bench.py's command-line contract on the host: a request for more than one
GPU ends at once with a one-line JSON error and exit status 2 (the fused
kernels emulate the peer ranks on one device)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = r.stdout.strip().splitlines()[-1]
    assert "one GPU" in json.loads(line)["error"]


def test_help_lists_the_switches():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--no-ect", "--no-cold", "--no-cpu-baseline",
                 "--copy-probe"):
        assert flag in r.stdout
