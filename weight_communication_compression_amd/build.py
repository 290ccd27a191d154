"""Build liblowbit.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m weight_communication_compression_amd.build [--force]

Every translation unit under ``csrc/`` is compiled separately (in parallel)
and linked into ``weight_communication_compression_amd/liblowbit.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblowbit.so")

SOURCES = ["api.cpp", "quantize_plain.hip", "quantize_ef.hip", "quantize_wdiff.hip",
           "quantize_ef21.hip", "quantize_hadamard.hip", "reduce.hip", "reduce_ef.hip", "reduce_mixed.hip",
           "dequant.hip", "measure.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Numerics: no FMA contraction, fp32 denormals kept, IEEE division; packed
# fp32 instructions disabled.
HIPFLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, extra: list[str], build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIPFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(force: bool = True, extra: list[str] | None = None, jobs: int | None = None,
          out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every HIP translation unit for gfx950 and link liblowbit.so.

    `extra` adds compiler flags (e.g. -D tuning macros); `out` and `build_dir`
    place a variant build elsewhere."""
    extra = list(extra or [])
    os.makedirs(build_dir, exist_ok=True)
    if not force and os.path.exists(out):
        newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
        newest = max(newest, os.path.getmtime(os.path.join(ROOT, "include", "lowbit.h")))
        if os.path.getmtime(out) >= newest:
            return out
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
