"""Build libxsymv.so for gfx950 with hipcc (in-tree, no JIT cache).

Each precision is its own translation unit so the units compile in parallel;
the shared library links them together.  Device code is compiled without
floating-point contraction (every fused multiply-add is written out) and
without packed-FP32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libxsymv.so")
UNITS = ["xsymv_host", "xsymv_prec_s", "xsymv_prec_d", "xsymv_prec_c", "xsymv_prec_z",
         "xsymv_prec_w", "xsymv_static"]
ARCH = os.environ.get("XSYMV_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _compile(unit: str, extra: list[str]) -> tuple[str, str]:
    src = os.path.join(CSRC, unit + ".hip")
    obj = os.path.join(BUILD, unit + ".o")
    r = subprocess.run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {unit}:\n{r.stderr}")
    return obj, r.stderr


def build(jobs: int | None = None, resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every unit and link ``libxsymv.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    jobs = jobs or min(len(UNITS), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda u: _compile(u, extra), UNITS))
    if verbose or resource_usage:
        for _, err in results:
            sys.stderr.write(err)
    tmp = LIB + f".tmp{os.getpid()}"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                        *[o for o, _ in results]], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--usage" in sys.argv, verbose="-v" in sys.argv))
