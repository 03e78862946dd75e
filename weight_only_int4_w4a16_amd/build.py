"""Build ``libw4a16.so`` (the C-ABI library) for gfx950 with hipcc, in the package folder.

Usage: ``python -m weight_only_int4_w4a16_amd.build`` (or ``build()`` from Python).
Each HIP source compiles to an object in ``_build/`` (in parallel), then one shared
library is linked next to this file. Flags: -O3, no fast-math (dequantization must round
exactly once), FP contraction off, and packed-FP32 instruction selection disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libw4a16.so")
SOURCES = ["w4a16_api.hip", "w4a16_pack.hip", "w4a16_decode.hip", "w4a16_tiled.hip",
           "w4a16_skinny.hip", "w4a16_w4a8.hip", "w4a16_probe.hip"] + [
    f"w4a16_decode_{a}_{f}.hip" for a in ("f16", "bf16") for f in ("asym", "sym", "nf4")] + [
    f"w4a16_tiled_{t}.hip" for t in ("large", "small", "smalldeep", "small2", "med")]
ARCH = os.environ.get("W4A16_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]


def _header_deps(path: str, seen=None) -> set:
    """The local headers a source includes, directly or through other headers."""
    seen = set() if seen is None else seen
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line.startswith('#include "'):
                continue
            name = line.split('"')[1]
            for d in (CSRC, os.path.join(ROOT, "include")):
                h = os.path.join(d, name)
                if os.path.exists(h) and h not in seen:
                    seen.add(h)
                    _header_deps(h, seen)
                    break
    return seen


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and os.path.exists(obj):
        t = os.path.getmtime(obj)
        deps = [os.path.join(CSRC, src), *_header_deps(os.path.join(CSRC, src))]
        if all(t > os.path.getmtime(d) for d in deps):
            return obj
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source (``incremental``: only those older than their object, or than a
    header) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda f: _compile(f, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
