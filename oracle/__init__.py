"""The oracle for the tiled dense GEMM path -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline leg
may import this package.  The GPU library (dense_gemm_fp8_amd) never imports
it, and it imports nothing from the GPU library.

Contents
  liboracle.so (oracle.c)  plain fp64 CPU GEMM C = A * B^T for bf16 and OCP e4m3
                           inputs, exact decoders, one-step bf16 rounding
  dense.py                 the same GEMM definition evaluated with exact fp64 decoding
                           and the BLAS fp64 matrix product, for full-size grids
  remap.py                 the chiplet-aware grid remap, written from the pages
  eq1.py                   the L2/LLC bandwidth model and its fit to Table 4
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (no fast-math: the
    k-ascending fp64 sums must stay as written)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_bf16_round_array.restype = None
        lib.oracle_bf16_round_array.argtypes = [p, p, i64]
        lib.oracle_gemm_bf16.restype = ctypes.c_int
        lib.oracle_gemm_bf16.argtypes = [i64, i64, i64, p, p, p, ctypes.c_int]
        lib.oracle_gemm_fp8.restype = ctypes.c_int
        lib.oracle_gemm_fp8.argtypes = [i64, i64, i64, p, p, ctypes.c_float, ctypes.c_float,
                                        p, ctypes.c_int]
        lib.oracle_gemm_bf16_pairs.restype = ctypes.c_int
        lib.oracle_gemm_bf16_pairs.argtypes = [i64, i64, i64, p, p, p, p, i64, p, ctypes.c_int]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_gemm_mxfp8.restype = ctypes.c_int
        lib.oracle_gemm_mxfp8.argtypes = [i64, i64, i64, p, p, p, p, p, ctypes.c_int]
        lib.oracle_gemm_mxfp8_pairs.restype = ctypes.c_int
        lib.oracle_gemm_mxfp8_pairs.argtypes = [i64, i64, i64, p, p, p, p, p, p, i64, p,
                                                ctypes.c_int]
        lib.oracle_gemm_fp8_pairs.restype = ctypes.c_int
        lib.oracle_gemm_fp8_pairs.argtypes = [i64, i64, i64, p, p, ctypes.c_float,
                                              ctypes.c_float, p, p, i64, p, ctypes.c_int]
        _lib = lib
    return _lib


def affinity_cores() -> int:
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_threads() -> int:
    """Worker threads: every core in the affinity mask, capped by OMP_NUM_THREADS
    when the environment sets it (a host that shares its cores between GPUs
    gives each GPU's processes that many)."""
    n = affinity_cores()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def e4m3_table() -> np.ndarray:
    """The 256 e4m3 code values (float64; NaN for the two NaN codes)."""
    lib = _load()
    return np.array([lib.oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)


def bf16_round(x) -> np.ndarray:
    """One round-to-nearest-even step from float64 to bfloat16 bits (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_round_array(_ptr(x), _ptr(out), x.size)
    return out


def _check(A, B, K, dt):
    if A.dtype != dt or B.dtype != dt:
        raise TypeError("expected %s inputs" % dt)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != K or B.shape[1] != K:
        raise ValueError("A must be [M,K] and B [N,K]")


def gemm_bf16(A: np.ndarray, B: np.ndarray, threads: int | None = None) -> np.ndarray:
    """fp64 reference of A·Bᵀ for bf16 bit arrays A [M,K], B [N,K]."""
    A = np.ascontiguousarray(A); B = np.ascontiguousarray(B)
    M, K = A.shape; N = B.shape[0]
    _check(A, B, K, np.uint16)
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_bf16(M, N, K, _ptr(A), _ptr(B), _ptr(out), threads or default_threads())
    if rc:
        raise RuntimeError("oracle_gemm_bf16 failed: %d" % rc)
    return out


def gemm_fp8(A: np.ndarray, B: np.ndarray, scale_a: float, scale_b: float,
             threads: int | None = None) -> np.ndarray:
    """fp64 reference of (sa·sb)·(A·Bᵀ) for e4m3 code arrays A [M,K], B [N,K]."""
    A = np.ascontiguousarray(A); B = np.ascontiguousarray(B)
    M, K = A.shape; N = B.shape[0]
    _check(A, B, K, np.uint8)
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_fp8(M, N, K, _ptr(A), _ptr(B), float(scale_a), float(scale_b),
                                 _ptr(out), threads or default_threads())
    if rc:
        raise RuntimeError("oracle_gemm_fp8 failed: %d" % rc)
    return out


def gemm_bf16_pairs(A, B, pm, pn, threads: int | None = None) -> np.ndarray:
    """fp64 reference values at the sampled coordinates (pm[i], pn[i])."""
    A = np.ascontiguousarray(A); B = np.ascontiguousarray(B)
    M, K = A.shape; N = B.shape[0]
    _check(A, B, K, np.uint16)
    pm = np.ascontiguousarray(pm, dtype=np.int64); pn = np.ascontiguousarray(pn, dtype=np.int64)
    out = np.empty(pm.shape, dtype=np.float64)
    rc = _load().oracle_gemm_bf16_pairs(M, N, K, _ptr(A), _ptr(B), _ptr(pm), _ptr(pn), pm.size,
                                        _ptr(out), threads or default_threads())
    if rc:
        raise RuntimeError("oracle_gemm_bf16_pairs failed: %d" % rc)
    return out


def gemm_fp8_pairs(A, B, scale_a, scale_b, pm, pn, threads: int | None = None) -> np.ndarray:
    A = np.ascontiguousarray(A); B = np.ascontiguousarray(B)
    M, K = A.shape; N = B.shape[0]
    _check(A, B, K, np.uint8)
    pm = np.ascontiguousarray(pm, dtype=np.int64); pn = np.ascontiguousarray(pn, dtype=np.int64)
    out = np.empty(pm.shape, dtype=np.float64)
    rc = _load().oracle_gemm_fp8_pairs(M, N, K, _ptr(A), _ptr(B), float(scale_a), float(scale_b),
                                       _ptr(pm), _ptr(pn), pm.size, _ptr(out),
                                       threads or default_threads())
    if rc:
        raise RuntimeError("oracle_gemm_fp8_pairs failed: %d" % rc)
    return out


def e8m0_value(e: int) -> float:
    return _load().oracle_e8m0_value(e)


def _check_mx(A, B, SA, SB, K):
    _check(A, B, K, np.uint8)
    if K % 32:
        raise ValueError("MXFP8 needs K % 32 == 0")
    if SA.dtype != np.uint8 or SB.dtype != np.uint8:
        raise TypeError("expected uint8 E8M0 scales")
    if SA.shape != (A.shape[0], K // 32) or SB.shape != (B.shape[0], K // 32):
        raise ValueError("SA must be [M,K/32] and SB [N,K/32]")


def gemm_mxfp8(A, B, SA, SB, threads: int | None = None) -> np.ndarray:
    """fp64 reference of the MXFP8 product: e4m3 codes A [M,K], B [N,K] with
    E8M0 block scales SA [M,K/32], SB [N,K/32] (one per 32 consecutive k)."""
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    SA, SB = np.ascontiguousarray(SA), np.ascontiguousarray(SB)
    M, K = A.shape; N = B.shape[0]
    _check_mx(A, B, SA, SB, K)
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_mxfp8(M, N, K, _ptr(A), _ptr(B), _ptr(SA), _ptr(SB), _ptr(out),
                                   threads or default_threads())
    if rc:
        raise RuntimeError("oracle_gemm_mxfp8 failed: %d" % rc)
    return out


def gemm_mxfp8_pairs(A, B, SA, SB, pm, pn, threads: int | None = None) -> np.ndarray:
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    SA, SB = np.ascontiguousarray(SA), np.ascontiguousarray(SB)
    M, K = A.shape; N = B.shape[0]
    _check_mx(A, B, SA, SB, K)
    pm = np.ascontiguousarray(pm, dtype=np.int64); pn = np.ascontiguousarray(pn, dtype=np.int64)
    out = np.empty(pm.shape, dtype=np.float64)
    rc = _load().oracle_gemm_mxfp8_pairs(M, N, K, _ptr(A), _ptr(B), _ptr(SA), _ptr(SB), _ptr(pm),
                                         _ptr(pn), pm.size, _ptr(out), threads or default_threads())
    if rc:
        raise RuntimeError("oracle_gemm_mxfp8_pairs failed: %d" % rc)
    return out
