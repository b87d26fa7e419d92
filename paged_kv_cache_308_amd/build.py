"""Build libpa.so (HIP for gfx950) in place: python -m paged_kv_cache_308_amd.build"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "libpa")
LIB = os.path.join(HERE, "libpa.so")

SOURCES = ["api.cpp", "host_api.cpp", "allocator.cpp", "cache_ops.hip", "decode_valu_f32.hip", "decode_valu_f16.hip",
           "decode_valu_bf16.hip", "decode_valu_fp8_f16.hip", "decode_valu_fp8_bf16.hip",
           "decode_mfma_f16.hip", "decode_mfma_bf16.hip", "multi_query_mfma_f16.hip",
           "multi_query_mfma_bf16.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# packed-fp32 instructions stay off: hipcc may form them from plain float code.
# fp32 division is correctly rounded (the E4M3 scatter picks codes from x / scale).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt"]


# Matrix-core units: keep MFMA accumulators in ordinary VGPRs.  By default the compiler
# places them in AGPRs and then moves them back and forth around every VALU touch
# (the online-softmax rescale), hundreds of v_accvgpr moves per loop iteration.
SOURCE_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for src in (
    "decode_mfma_f16.hip", "decode_mfma_bf16.hip", "multi_query_mfma_f16.hip", "multi_query_mfma_bf16.hip")}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra=(), jobs: int = 8, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(extra=sys.argv[1:])
