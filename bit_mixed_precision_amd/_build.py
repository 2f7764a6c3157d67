"""Build libbq.so in-tree: hipcc for gfx950 only, one object per source file
(compiled in parallel), then a shared link; and libbq_calib.so, the
benchmark's measurement kernels (not part of the library)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_HERE, "csrc")
OBJDIR = os.path.join(_HERE, "_build")
LIB = os.path.join(_HERE, "libbq.so")
# measurement kernels for the benchmark's achievable ceilings (not the library)
CALIB_SRC = os.path.join(CSRC, "calib", "calib.hip")
CALIB_LIB = os.path.join(_HERE, "libbq_calib.so")
SOURCES = ["api.hip", "quantize.hip", "pack.hip", "gemv.hip", "gemv_nf4.hip", "gemm_stream.hip", "gemm_tiled.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: with the accumulation
    # registers the allocator shuffled accumulators between loop halves
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_calib()
    return LIB


def build_calib() -> str:
    tmp = CALIB_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", CALIB_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for calib.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


if __name__ == "__main__":
    print(build())
