"""Build libhkg.so (the gfx950 kernels + C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhkg.so")
SOURCES = [os.path.join(CSRC, "gemm_kernels.hip"), os.path.join(CSRC, "hkg_api.cpp"),
           os.path.join(CSRC, "launch.cpp"), os.path.join(CSRC, "remap_model.cpp"),
           os.path.join(CSRC, "tune.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep hipcc from forming packed fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# The compiler's per-kernel resource report (registers, scratch, spills).
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def scratch_users(report: str) -> list[tuple[str, str, int]]:
    """(kernel, item, value) for every kernel that the report shows using
    scratch memory or spilling registers.  The GEMM kernels keep their whole
    accumulator tile in registers; if the compiler ever demotes it to scratch
    the kernel still computes the right answer, only 10-60x slower, so the
    build treats that as an error."""
    bad, fn = [], None
    for line in report.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            fn = m.group(1)
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and fn and int(m.group(2)) > 0:
            bad.append((fn, m.group(1), int(m.group(2))))
    return bad


def waterfall_loops(asm: str) -> list[tuple[str, str]]:
    """(function, loop label) of every loop in a gfx950 assembly listing that
    branches back on a non-empty exec mask (s_cbranch_execnz) and issues a
    buffer load.  The compiler emits such a loop when an operand that must be
    scalar (a buffer load's soffset or resource) is held in a vector register:
    it loads once per distinct lane value.  The GEMM kernels pass only uniform
    values there, so any such loop is a code-generation regression (it once
    cost the e4m3 ping-pong 9 % of its cycles per K step)."""
    found, fn, labels, body_start = [], None, {}, {}
    lines = asm.splitlines()
    for i, line in enumerate(lines):
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", line)
        if m and not m.group(1).startswith(".L"):
            fn, labels = m.group(1), {}
            continue
        m = re.match(r"^(\.LBB\w+):", line)
        if m:
            labels[m.group(1)] = i
            continue
        m = re.match(r"\s+s_cbranch_execnz\s+(\.LBB\w+)", line)
        if m and m.group(1) in labels:
            body = lines[labels[m.group(1)]:i]
            if any(re.match(r"\s+buffer_load", x) for x in body):
                found.append((fn, m.group(1)))
    return found


def device_asm(out: str) -> None:
    """Compile the kernels' source to gfx950 assembly (device code only) with
    the library's flags, into `out`."""
    cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(CSRC, "gemm_kernels.hip"), "-I", os.path.join(ROOT, "include"), "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-3000:])


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source into dense_gemm_fp8_amd/libhkg.so (always rebuilds);
    fails if a kernel uses scratch memory or spills registers."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, RESOURCE_REMARKS, *(extra or []), "-shared", "-x", "hip",
           *SOURCES, "-I", os.path.join(ROOT, "include"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    other = [ln for ln in res.stderr.splitlines()
             if "kernel-resource-usage" not in ln and "packed-fp32-ops" not in ln]
    if other and (verbose or res.returncode != 0):
        print("\n".join(other), file=sys.stderr, flush=True)
    if res.returncode != 0:
        raise subprocess.CalledProcessError(res.returncode, cmd)
    bad = scratch_users(res.stderr)
    if bad:
        os.unlink(tmp)
        raise RuntimeError("kernels using scratch memory: %s" % bad)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
