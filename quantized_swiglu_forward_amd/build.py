"""Build the HIP library ``libswiglu_q.so`` in-tree with hipcc for gfx950.

Usage: ``python -m quantized_swiglu_forward_amd.build`` (or ``build_library()``).
Each source compiles to its own object in parallel, then one link step.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libswiglu_q.so")
SOURCES = ["swq_api.hip", "swq_prefill.hip", "swq_gemv.hip", "swq_gemv_f16.hip"]
# measurement yardsticks for the benchmark only (a library of their own)
PROBE_LIB = os.path.join(PKG, "libswq_probe.so")
PROBE_SOURCES = ["swq_probe.hip"]
# debug build of the same library whose kernels poison their LDS before use
# (read by a GPU test only)
POISON_LIB = os.path.join(PKG, "libswiglu_q_ldspoison.so")
POISON_FLAGS = ["-DSWQ_LDS_POISON"]
ARCH = os.environ.get("SWIGLU_Q_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # packed float32 instructions are disabled on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(job) -> str:
    src, extra = job if isinstance(job, tuple) else (job, [])
    tag = "_poison" if extra else ""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source and link ``libswiglu_q.so``, its LDS-poison
    debug twin and the benchmark's ``libswq_probe.so`` (all objects in
    parallel); returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = SOURCES + PROBE_SOURCES + [(src, POISON_FLAGS) for src in SOURCES]
    workers = min(len(jobs), max(1, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, jobs))
    n, m = len(SOURCES), len(PROBE_SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + m], PROBE_LIB)
    _link(objs[n + m:], POISON_LIB)
    if verbose:
        for lib in (LIB, PROBE_LIB, POISON_LIB):
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
