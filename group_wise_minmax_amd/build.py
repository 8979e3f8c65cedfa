"""Build liblbq.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m group_wise_minmax_amd.build        # or __graft_entry__.build()

Every call recompiles every source.  The shared library lands next to this
file, where the Python binding loads it.  The benchmark's streaming-read
ceiling (bench_stream.hip, not part of liblbq) is built beside bench.py.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblbq.so")
ARCH = "gfx950"

COMMON = [
    "-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-I", CSRC, "-I", INCLUDE,
]
# Quantize/dequantize must be bit-exact: one IEEE op per step, no contraction.
# The small-batch kernel accumulates its MFMAs in ordinary registers: its
# epilogue reads every accumulator once per group, which the accumulation
# registers would cost an extra move each.
PER_FILE = {"k_quant.hip": ["-ffp-contract=off"],
            "k_skinny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["lbq_api.cpp", "k_quant.hip", "k_gemv1.hip", "k_skinny.hip", "k_gemm_fwd.hip", "k_bwd.hip", "k_lora.hip",
           "k_noalloc.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# The benchmark's streaming-read ceiling (not part of liblbq), beside bench.py.
BENCH_STREAM_SRC = os.path.join(ROOT, "bench_stream.hip")
BENCH_STREAM_LIB = os.path.join(ROOT, "libbench_stream.so")


def _build_bench_stream() -> str:
    tmp = BENCH_STREAM_LIB + ".tmp"
    cmd = [hipcc(), *COMMON, "-shared", BENCH_STREAM_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, BENCH_STREAM_LIB)
    return BENCH_STREAM_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES) + 1)) as ex:
        bench_lib = ex.submit(_build_bench_stream)
        objs = list(ex.map(_compile, SOURCES))
        bench_lib.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
