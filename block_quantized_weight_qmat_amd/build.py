"""Build libqmat.so (gfx950) from csrc/ with hipcc, in-tree, and beside it
libqmat_micro.so, the measured-peak kernels that only the benchmark loads.

    python -m block_quantized_weight_qmat_amd.build

Every source is compiled for gfx950 only, without fp contraction (the
kernels call fmaf where a fused multiply-add is meant, and the quantizers
must round exactly as written) and without packed fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmat.so")
MICRO_LIB = os.path.join(PKG, "libqmat_micro.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quantize.hip", "gemv.hip", "decode.hip", "gemm.hip", "qmat_api.cpp"]
MICRO_SOURCES = ["micro.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the GEMM epilogue reads every value,
    # and results in AGPRs would cost a v_accvgpr_read each
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    # -z defs: a kernel whose host stub was not emitted (an instantiation the
    # host pass dropped) is an error here, not a library that fails to load
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + MICRO_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], MICRO_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
