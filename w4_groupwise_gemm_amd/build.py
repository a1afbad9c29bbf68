"""Build step: compile the HIP kernels and the C ABI into ``libw4gemm.so`` (gfx950 only).

Run ``python -m w4_groupwise_gemm_amd.build`` (or ``__graft_entry__.build()``).  Objects go to
``w4_groupwise_gemm_amd/_build``; the library is written next to this file.
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
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw4gemm.so")
PROBE_LIB = os.path.join(HERE, "libw4probe.so")  # measurement support (read/copy/empty kernels)

SOURCES = ["api.hip", "stream.hip", "narrow.hip", "splitk.hip", "wide.hip", "repack.cpp"]
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")

# Packed-FP32 instructions are disabled for all device code.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE_FLAGS if src.endswith(".hip") else []) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    shutil.move(tmp, out)


def build(verbose: bool = False, jobs: int = 6) -> str:
    """Compile every source (always, even if a library exists) and link libw4gemm.so and the
    measurement-support libw4probe.so."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
