"""bench.py on the GPU: a short run prints one JSON line that carries the
contract's keys, a roofline for the dominant kernel, per-op median and
minimum times, and the cold-cache timing of each op; and the two probe modes
behind the profiles (the matrix-core ceiling and the byte-counter copy)."""
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


def _bench_json(args, timeout=110):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.strip().splitlines() if x.startswith("{")]
    assert len(lines) == 1
    return json.loads(lines[0])


def test_mfma_ceiling_mode():
    """bench.py --mfma-ceiling (the register-only matrix-core probe behind the
    clock evidence): every form reports a rate, a clock and a fraction of the
    peak at that clock that a real chip can reach."""
    say("bench.py --mfma-ceiling")
    rows = _bench_json(["--mfma-ceiling"])["mfma_ceiling"]
    assert len(rows) == 16
    forms = {(r["dtype"], r["mfma"], r["waves_per_simd"], r["operands"]) for r in rows}
    assert len(forms) == 16
    for r in rows:
        assert r["tflops"] > 0 and 0.3 < r["clock_ghz"] < 3.0, r
        assert 0 < r["frac_at_clock"] <= 1.02, r


def test_copy_probe_mode():
    """bench.py --copy-probe (the known-size copy that calibrates the HBM
    byte counters) copies what it says and reports the sizes."""
    say("bench.py --copy-probe 16")
    d = _bench_json(["--copy-probe", "16"])
    assert d == {"copy_probe_bytes_read": 16 << 20, "copy_probe_bytes_written": 16 << 20,
                 "dispatches": 3}
