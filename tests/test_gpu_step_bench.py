"""bench.py on the GPU: a short run prints one JSON line that carries the
contract's keys, a roofline for the dominant kernel, per-op median and
minimum times, and the cold-cache timing of each op."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_short_bench_line():
    say("bench.py --steps 3 --warmup 1 --no-ect --no-cpu-baseline")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-ect", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.strip().splitlines() if x.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    names = ("ag_gemm", "gemm_rs", "moe_gather_gemm", "moe_gemm_scatter")
    for n in names:
        op = d["ops"][n]
        assert 0 < op["min_ms"] <= op["median_ms"]
        assert d["cold_ms"][n] > 0
    rf = d["roofline"]
    assert rf["kernel"] in names and rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s"
    assert 0 < rf["frac"] < 1 and abs(rf["achieved"] / rf["peak"] - rf["frac"]) < 1e-3
