"""Build tests/c/abi_extremes: every entry point of libhkg driven with extreme
arguments (abi_extremes.c), linked with the library's sources compiled afresh
with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only.
Device code is built as usual and never run: the driver needs no GPU, and it
runs on the CPU host only."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_extremes.c")
EXE = os.path.join(HERE, "abi_extremes")
SANITIZERS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"]


def commands(out: str, objdir: str) -> list[list[str]]:
    """Compile lines for the library sources (each sanitizer option behind
    -Xarch_host, so only host code is instrumented), the driver, and the
    link."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from dense_gemm_fp8_amd import build as lib_build
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    llvm = os.path.join(rocm, "lib", "llvm", "bin")
    host_only = [x for f in SANITIZERS for x in ("-Xarch_host", f)]
    flags = [f for f in lib_build.HIPCC_FLAGS if f != "-O3"]
    cmds, objs = [], []
    for src in lib_build.SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmds.append([lib_build.hipcc(), *flags, "-O1", "-g", *host_only, "-c", "-x", "hip", src,
                     "-I", os.path.join(ROOT, "include"), "-o", obj])
        objs.append(obj)
    drv = os.path.join(objdir, "abi_extremes.o")
    cmds.append([os.path.join(llvm, "clang"), "-std=c99", "-O1", "-g", "-Wall", "-Werror", *SANITIZERS,
                 "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                 "-I", os.path.join(ROOT, "include"), "-c", SRC, "-o", drv])
    cmds.append([os.path.join(llvm, "clang++"), *SANITIZERS[:2], *objs, drv, "-o", out,
                 "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                 "-Wl,-rpath," + os.path.join(rocm, "lib")])
    return cmds


def build(out: str = EXE) -> str:
    with tempfile.TemporaryDirectory() as tmp:
        for cmd in commands(out, tmp):
            subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    return out


if __name__ == "__main__":
    print(build())
