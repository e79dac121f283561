"""Build the HIP library libdq.so in-tree for gfx950.

``python -m calibration_free_bit_amd.build`` (or ``build()``) compiles
``csrc/`` with hipcc into ``calibration_free_bit_amd/_lib/libdq.so``. The
kernel file is compiled once per element grid, in parallel.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libdq.so")
ARCH = "gfx950"


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        # no packed-fp32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the first 14 dwords of kernel arguments arrive in SGPRs at wave
        # launch instead of through a scalar load (gfx950 kernarg preload)
        "-mllvm", "-amdgpu-kernarg-preload-count=14",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _units():
    k = os.path.join(CSRC, "dq_kernels.hip")
    return [
        ("dq_api.o", os.path.join(CSRC, "dq_api.hip"), []),
        ("dq_kernels_int4.o", k, ["-DDQ_GRID_INST=dq::kGridInt4"]),
        ("dq_kernels_e2m1.o", k, ["-DDQ_GRID_INST=dq::kGridE2M1"]),
        ("dq_kernels_int8.o", k, ["-DDQ_GRID_INST=dq::kGridInt8"]),
        ("dq_kernels_e4m3.o", k, ["-DDQ_GRID_INST=dq::kGridE4M3"]),
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every unit and link libdq.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for obj, src, defs in _units():
        out = os.path.join(BUILD_DIR, obj)
        jobs.append((out, [cc, *common_flags(), *defs, *extra_flags, "-c", src, "-o", out]))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda j: _run(j[1], verbose), jobs))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *[j[0] for j in jobs]], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
