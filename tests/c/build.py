"""Build tests/c/gemm_c_api (a plain C99 caller of libhkg) with gcc against
include/hkg.h, the HIP runtime API and dense_gemm_fp8_amd/libhkg.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "gemm_c_api.c")
EXE = os.path.join(HERE, "gemm_c_api")


def command(out: str = EXE) -> list[str]:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib = os.path.join(ROOT, "dense_gemm_fp8_amd")
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", out,
            "-L", lib, "-lhkg", "-Wl,-rpath,$ORIGIN/../../dense_gemm_fp8_amd", "-Wl,-rpath," + lib,
            "-L", os.path.join(rocm, "lib"), "-lamdhip64",
            "-Wl,-rpath," + os.path.join(rocm, "lib")]


def build(out: str = EXE) -> str:
    subprocess.run(command(out), check=True)
    return out

