"""Build libfluxmi.so (HIP, gfx950 only) in-tree.

Every source under csrc/ is compiled by hipcc for gfx950 and linked into one
shared library next to this file, which the Python binding loads.  Packed
fp32 VALU ops are disabled for every device compile.  The compiler's
per-kernel register and scratch figures are kept in
_build/kernel_resources.json, which the CPU tests check.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfluxmi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.json")


def _resources(remarks: str) -> list:
    """Per-kernel register and scratch use from hipcc's resource remarks."""
    out, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]):\s*(\S+)", line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = {"name": val}
            out.append(cur)
        elif cur is not None:
            cur[{"VGPRs": "vgpr", "AGPRs": "agpr"}.get(key, "scratch")] = int(val)
    return out


def _compile(src: str):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    with open(RESOURCES, "w") as f:
        json.dump([k for _, ks in done for k in ks], f, indent=0)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
