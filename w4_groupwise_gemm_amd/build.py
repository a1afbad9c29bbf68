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

# (source, extra defines, object) -- stream.hip is compiled once per code width and epilogue,
# narrow.hip once per code width
STREAM_PARTS = [("stream.hip", [f"-DW4_STREAM_BITS={b}", f"-DW4_STREAM_EPI={e}"], f"stream_b{b}_e{e}.o")
                for b in (4, 5) for e in (0, 1, 2)]
NARROW_PARTS = [("narrow.hip", [f"-DW4_NARROW_BITS={b}"], f"narrow_b{b}.o") for b in (4, 5)]
REGRING_PARTS = [("regring.hip", [f"-DW4_REGRING_BITS={b}"], f"regring_b{b}.o") for b in (4, 5)]
SOURCES = STREAM_PARTS + NARROW_PARTS + REGRING_PARTS + ["api.hip", "splitk.hip", "wide.hip", "bf16.hip", "a8.hip", "repack.cpp", "graphs.cpp"]
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")

# Packed-FP32 instructions are disabled for all device code.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(item) -> str:
    src, defines, objname = item if isinstance(item, tuple) else (item, [], os.path.splitext(item)[0] + ".o")
    obj = os.path.join(BUILD, objname)
    cmd = [HIPCC] + COMMON + (DEVICE_FLAGS if src.endswith(".hip") else []) + list(defines) + \
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


def build(verbose: bool = False, jobs: int = 8) -> str:
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
