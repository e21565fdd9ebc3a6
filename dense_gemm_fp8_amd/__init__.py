"""dense_gemm_fp8_amd -- Python binding of libhkg, the MI355X (gfx950) tiled GEMM.

    C[M,N] = A[M,K] · B[N,K]ᵀ     (bf16, OCP e4m3 or MXFP8 inputs, fp32 accumulate, bf16 out)

The C ABI (include/hkg.h) is the product; this module only marshals
arguments.  The functions with the C names (hkg_gemm_bf16, ...) take integers
for device pointers and the stream, exactly like the C entry points.  The
torch helpers (gemm_bf16, gemm_fp8, gemm_mxfp8, mx_pack_scales,
remap_tiles_device) take torch tensors that
already live on the GPU; torch is used for device memory and streams only,
every step of the GEMM runs in the library's own kernels.

The shared library is built in-tree by dense_gemm_fp8_amd/build.py (or
__graft_entry__.build()).  If it is missing, loading raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhkg.so")

HKG_OK = 0
HKG_ERR_NULL = -1
HKG_ERR_SHAPE = -2
HKG_ERR_ALIGN = -3
HKG_ERR_SIZE = -4
HKG_ERR_OPTS = -5
HKG_ERR_DEVICE = -6
HKG_ERR_LAUNCH = -7
HKG_ERR_OVERLAP = -8

HKG_REMAP_DEFAULT = 0
HKG_REMAP_ROW_MAJOR = 1
HKG_REMAP_XCD = 2

HKG_SCHED_DEFAULT = 0
HKG_SCHED_PINGPONG = 1
HKG_SCHED_LOCKSTEP = 2
HKG_SCHED_INTERLEAVE = 3
HKG_SCHED_INTERLEAVE_128 = 4
HKG_SCHED_INTERLEAVE_192 = 5

HKG_MX_OPERAND_A = 0
HKG_MX_OPERAND_B = 1

# exported symbols, in the order include/hkg.h declares them
EXPORTS = (
    "hkg_gemm_bf16",
    "hkg_gemm_fp8",
    "hkg_gemm_bf16_ex",
    "hkg_gemm_fp8_ex",
    "hkg_gemm_mxfp8",
    "hkg_gemm_mxfp8_ex",
    "hkg_mx_packed_scale_bytes",
    "hkg_mx_pack_scales",
    "hkg_default_remap",
    "hkg_launch_plan",
    "hkg_remap_model",
    "hkg_remap_candidates",
    "hkg_tune_remap",
    "hkg_remap_tile",
    "hkg_remap_tiles_device",
    "hkg_probe_xcd",
    "hkg_status_string",
    "hkg_last_hip_error",
)


class hkg_gemm_opts(ctypes.Structure):
    _fields_ = [("remap", ctypes.c_int32), ("W", ctypes.c_int32), ("C", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("trace", ctypes.c_void_p),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64)]


class hkg_launch_plan_t(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32), ("schedule", ctypes.c_int32 * 2),
                ("tile", ctypes.c_int32 * 2), ("rows", ctypes.c_int64 * 2),
                ("grid", ctypes.c_int64 * 2), ("W", ctypes.c_int32 * 2), ("C", ctypes.c_int32 * 2)]


class HkgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s failed: %d (%s)" % (where, status, status_string(status))
        if status == HKG_ERR_LAUNCH:
            msg += ", hip error %d" % hkg_last_hip_error()
        super().__init__(msg)


_lib = None


def load() -> ctypes.CDLL:
    """Load libhkg.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime (same soname as ROCm's).  Loading torch
    # first makes libhkg bind to that runtime, so kernels launch on the streams
    # and device memory torch hands out; loading libhkg first would put two HIP
    # runtimes in the process.
    try:
        import torch  # noqa: F401
    except ImportError:  # plain C-ABI use without torch
        pass
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libhkg.so is not built (run python dense_gemm_fp8_amd/build.py "
                           "or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, p, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    popts = ctypes.POINTER(hkg_gemm_opts)
    sig = {
        "hkg_gemm_bf16": [i64, i64, i64, p, p, p, p, p],
        "hkg_gemm_fp8": [i64, i64, i64, p, p, f32, f32, p, p, p],
        "hkg_gemm_bf16_ex": [i64, i64, i64, p, p, p, p, p, popts],
        "hkg_gemm_fp8_ex": [i64, i64, i64, p, p, f32, f32, p, p, p, popts],
        "hkg_gemm_mxfp8": [i64, i64, i64, p, p, p, p, p, p, p],
        "hkg_gemm_mxfp8_ex": [i64, i64, i64, p, p, p, p, p, p, p, popts],
        "hkg_mx_packed_scale_bytes": [i64, i64],
        "hkg_mx_pack_scales": [i32, i64, i64, p, p, p],
        "hkg_default_remap": [i64, i64, i64, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)],
        "hkg_launch_plan": [i64, i64, i64, i32, ctypes.POINTER(hkg_gemm_opts),
                            ctypes.POINTER(hkg_launch_plan_t)],
        "hkg_remap_model": [i64, i64, i32, i32, i64, i32, ctypes.POINTER(ctypes.c_double),
                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)],
        "hkg_remap_candidates": [i64, i64, i64, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)],
        "hkg_tune_remap": [i64, i64, i64, i32, p, p, p, i32, popts, ctypes.POINTER(f32), popts,
                           ctypes.POINTER(f32), ctypes.POINTER(i32), p],
        "hkg_remap_tile": [i64, i64, i32, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)],
        "hkg_remap_tiles_device": [i64, i64, i32, i32, p, p],
        "hkg_probe_xcd": [i64, i32, i32, p, p],
        "hkg_status_string": [ctypes.c_int],
        "hkg_last_hip_error": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = {"hkg_status_string": ctypes.c_char_p,
                      "hkg_mx_packed_scale_bytes": ctypes.c_int64}.get(name, ctypes.c_int)
    _lib = lib
    return lib


# ---- the C entry points, same names and arguments ---------------------------------

def hkg_gemm_bf16(M, N, K, A, B, C, C_f32, stream) -> int:
    return load().hkg_gemm_bf16(M, N, K, A, B, C, C_f32, stream)


def hkg_gemm_fp8(M, N, K, A, B, scale_a, scale_b, C, C_f32, stream) -> int:
    return load().hkg_gemm_fp8(M, N, K, A, B, scale_a, scale_b, C, C_f32, stream)


def hkg_gemm_bf16_ex(M, N, K, A, B, C, C_f32, stream, opts) -> int:
    return load().hkg_gemm_bf16_ex(M, N, K, A, B, C, C_f32, stream,
                                   ctypes.byref(opts) if opts is not None else None)


def hkg_gemm_fp8_ex(M, N, K, A, B, scale_a, scale_b, C, C_f32, stream, opts) -> int:
    return load().hkg_gemm_fp8_ex(M, N, K, A, B, scale_a, scale_b, C, C_f32, stream,
                                  ctypes.byref(opts) if opts is not None else None)


def hkg_gemm_mxfp8(M, N, K, A, B, SA_packed, SB_packed, C, C_f32, stream) -> int:
    return load().hkg_gemm_mxfp8(M, N, K, A, B, SA_packed, SB_packed, C, C_f32, stream)


def hkg_gemm_mxfp8_ex(M, N, K, A, B, SA_packed, SB_packed, C, C_f32, stream, opts) -> int:
    return load().hkg_gemm_mxfp8_ex(M, N, K, A, B, SA_packed, SB_packed, C, C_f32, stream,
                                    ctypes.byref(opts) if opts is not None else None)


def hkg_mx_packed_scale_bytes(rows, K) -> int:
    return load().hkg_mx_packed_scale_bytes(rows, K)


def hkg_mx_pack_scales(operand, rows, K, scales, packed, stream) -> int:
    return load().hkg_mx_pack_scales(operand, rows, K, scales, packed, stream)


def hkg_default_remap(M, N, K, dtype):
    """-> (status, W, C)."""
    W, C = ctypes.c_int32(), ctypes.c_int32()
    rc = load().hkg_default_remap(M, N, K, dtype, ctypes.byref(W), ctypes.byref(C))
    return rc, W.value, C.value


def launch_plan(M, N, K, dtype, opts=None):
    """What a GEMM call launches (hkg_launch_plan): (status, [launch dicts])
    with keys schedule, tile, rows, grid, W, C; dtype 0 bf16, 1 e4m3, 2 MXFP8."""
    pl = hkg_launch_plan_t()
    rc = load().hkg_launch_plan(M, N, K, dtype, ctypes.byref(opts) if opts is not None else None,
                                ctypes.byref(pl))
    out = [dict(schedule=pl.schedule[i], tile=pl.tile[i], rows=pl.rows[i], grid=pl.grid[i],
                W=pl.W[i], C=pl.C[i]) for i in range(pl.launches)] if rc == HKG_OK else []
    return rc, out


def hkg_remap_model(Gm, Gn, W, C, panel_bytes, per_xcd=32):
    """-> (status, l2_hit, llc_hit, eq1_bw_tbs) of the library's cache model."""
    l2, llc, bw = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = load().hkg_remap_model(Gm, Gn, W, C, panel_bytes, per_xcd, ctypes.byref(l2),
                                ctypes.byref(llc), ctypes.byref(bw))
    return rc, l2.value, llc.value, bw.value


def hkg_remap_candidates(M, N, K, dtype, max_out=48):
    """-> (status, [(W, C, eq1_bw_tbs), ...] best first, count)."""
    W = (ctypes.c_int32 * max(max_out, 1))()
    C = (ctypes.c_int32 * max(max_out, 1))()
    bw = (ctypes.c_double * max(max_out, 1))()
    n = ctypes.c_int32()
    rc = load().hkg_remap_candidates(M, N, K, dtype, max_out, W, C, bw, ctypes.byref(n))
    got = min(n.value, max_out) if rc == HKG_OK else 0
    return rc, [(W[i], C[i], bw[i]) for i in range(got)], n.value


HKG_TUNE_MAX_CANDIDATES = 8


def hkg_tune_remap(M, N, K, dtype, A, B, C, launches, best, stream):
    """-> (status, best_ms, [(opts, ms) of every configuration timed]); fills
    the hkg_gemm_opts `best`."""
    ms = ctypes.c_float()
    tried = (hkg_gemm_opts * HKG_TUNE_MAX_CANDIDATES)()
    tried_ms = (ctypes.c_float * HKG_TUNE_MAX_CANDIDATES)()
    n = ctypes.c_int32()
    rc = load().hkg_tune_remap(M, N, K, dtype, A, B, C, launches, ctypes.byref(best),
                               ctypes.byref(ms), tried, tried_ms, ctypes.byref(n), stream)
    got = n.value if rc == HKG_OK else 0
    return rc, ms.value, [(tried[i], tried_ms[i]) for i in range(got)]


def hkg_remap_tile(Gm, Gn, W, C, b):
    """-> (status, tile_m, tile_n)."""
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    rc = load().hkg_remap_tile(Gm, Gn, W, C, b, ctypes.byref(tm), ctypes.byref(tn))
    return rc, tm.value, tn.value


def hkg_remap_tiles_device(Gm, Gn, W, C, out, stream) -> int:
    return load().hkg_remap_tiles_device(Gm, Gn, W, C, out, stream)


def hkg_probe_xcd(workgroups, full_lds, spin_cycles, out, stream) -> int:
    return load().hkg_probe_xcd(workgroups, full_lds, spin_cycles, out, stream)


def hkg_status_string(status: int) -> str:
    return load().hkg_status_string(status).decode()


def hkg_last_hip_error() -> int:
    return load().hkg_last_hip_error()


status_string = hkg_status_string


# ---- torch marshalling helpers ------------------------------------------------------

def make_opts(remap=HKG_REMAP_DEFAULT, W=0, C=0, schedule=HKG_SCHED_DEFAULT,
              trace=None, lda=0, ldb=0, ldc=0) -> hkg_gemm_opts:
    """Options of the _ex entry points; trace: None or a device pointer (int) /
    uint64 GPU tensor for the per-workgroup time record; lda / ldb / ldc: row
    pitches in elements (0 = dense)."""
    if trace is not None and not isinstance(trace, int):
        trace = _dev_ptr(trace, "trace")
    return hkg_gemm_opts(remap, W, C, schedule, trace, lda, ldb, ldc)


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _matrix(t, name):
    """(device pointer, row pitch in elements) of a 2-D GPU tensor whose rows are
    contiguous (stride 1 along the row); the pitch is its row stride, which may
    exceed the row length (a view of a wider matrix, or padded rows)."""
    if t is None:
        return None, 0
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    rows, cols = t.shape
    if t.is_contiguous():
        return t.data_ptr(), cols
    if t.stride(1) != 1 or t.stride(0) < cols:
        raise ValueError("%s must have contiguous rows (stride 1 along a row)" % name)
    return t.data_ptr(), t.stride(0)


def _operands(A, B, C, C_f32, opts, M, N, K):
    """Pointers of A, B, C, C_f32 and the options with their row pitches."""
    pA, lda = _matrix(A, "A")
    pB, ldb = _matrix(B, "B")
    pC, ldc = _matrix(C, "C")
    pF, ldf = _matrix(C_f32, "C_f32")
    if C_f32 is not None and ldf != ldc:
        raise ValueError("C and C_f32 must have the same row pitch")
    return pA, pB, pC, pF, _with_pitches(opts, lda, ldb, ldc, dict(lda=K, ldb=K, ldc=N))


def _with_pitches(opts, lda, ldb, ldc, dense):
    """opts with the tensors' row pitches filled in where opts leaves them 0;
    None when every pitch is the dense one and no opts were given."""
    want = dict(lda=lda, ldb=ldb, ldc=ldc)
    if opts is None:
        if all(want[k] == dense[k] for k in want):
            return None
        opts = make_opts()
    out = hkg_gemm_opts(opts.remap, opts.W, opts.C, opts.schedule, opts.trace, opts.lda, opts.ldb,
                        opts.ldc)
    for k, v in want.items():
        given = getattr(out, k)
        if given == 0:
            setattr(out, k, v)
        elif v != dense[k] and given != v:
            raise ValueError("opts.%s = %d disagrees with the tensor's row stride %d" % (k, given, v))
    return out


def gemm_bf16(A, B, C=None, C_f32=None, opts=None, stream=None):
    """C[M,N] (bf16) = A[M,K] · B[N,K]ᵀ for bf16 GPU tensors; returns C.  Each
    2-D tensor needs contiguous rows; a row stride beyond the row length (a view
    of a wider matrix, or padded rows) is passed as its pitch (lda / ldb / ldc)."""
    import torch
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be torch.bfloat16")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A is [M,K] and B is [N,K]")
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if tuple(C.shape) != (M, N) or C.dtype != torch.bfloat16:
        raise ValueError("C must be a [M,N] bfloat16 tensor")
    if C_f32 is not None and (tuple(C_f32.shape) != (M, N) or C_f32.dtype != torch.float32):
        raise ValueError("C_f32 must be a [M,N] float32 tensor")
    pA, pB, pC, pF, opts = _operands(A, B, C, C_f32, opts, M, N, K)
    rc = hkg_gemm_bf16_ex(M, N, K, pA, pB, pC, pF, _stream_handle(stream), opts)
    if rc != HKG_OK:
        raise HkgError(rc, "hkg_gemm_bf16_ex")
    return C


def gemm_fp8(A, B, scale_a, scale_b, C=None, C_f32=None, opts=None, stream=None):
    """C[M,N] (bf16) = bf16(sa·sb · A[M,K] · B[N,K]ᵀ) for e4m3 code tensors
    (torch.uint8 or torch.float8_e4m3fn) on the GPU; returns C.  Row strides
    become pitches as in gemm_bf16."""
    import torch
    ok = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    if A.dtype not in ok or B.dtype not in ok:
        raise TypeError("A and B must hold e4m3 bytes (uint8 or float8_e4m3fn)")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A is [M,K] and B is [N,K]")
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if tuple(C.shape) != (M, N) or C.dtype != torch.bfloat16:
        raise ValueError("C must be a [M,N] bfloat16 tensor")
    if C_f32 is not None and (tuple(C_f32.shape) != (M, N) or C_f32.dtype != torch.float32):
        raise ValueError("C_f32 must be a [M,N] float32 tensor")
    pA, pB, pC, pF, opts = _operands(A, B, C, C_f32, opts, M, N, K)
    rc = hkg_gemm_fp8_ex(M, N, K, pA, pB, float(scale_a), float(scale_b), pC, pF,
                         _stream_handle(stream), opts)
    if rc != HKG_OK:
        raise HkgError(rc, "hkg_gemm_fp8_ex")
    return C


def mx_pack_scales(scales, operand, packed=None, stream=None):
    """Pack one MXFP8 operand's E8M0 scales (uint8 GPU tensor [rows, K/32]) into
    the kernel's order (hkg_mx_pack_scales); returns the packed uint8 tensor."""
    import torch
    if scales.dtype != torch.uint8 or scales.dim() != 2:
        raise TypeError("scales must be a 2-D uint8 tensor [rows, K/32]")
    rows, nblk = scales.shape
    K = 32 * nblk
    nbytes = hkg_mx_packed_scale_bytes(rows, K)
    if nbytes < 0:
        raise HkgError(nbytes, "hkg_mx_packed_scale_bytes")
    if packed is None:
        packed = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=scales.device)
    if packed.dtype != torch.uint8 or packed.numel() < nbytes:
        raise ValueError("packed must be a uint8 tensor of at least %d bytes" % nbytes)
    rc = hkg_mx_pack_scales(operand, rows, K, _dev_ptr(scales, "scales"), _dev_ptr(packed, "packed"),
                            _stream_handle(stream))
    if rc != HKG_OK:
        raise HkgError(rc, "hkg_mx_pack_scales")
    return packed


def gemm_mxfp8(A, B, SA_packed, SB_packed, C=None, C_f32=None, opts=None, stream=None):
    """C[M,N] (bf16) = A[M,K] · B[N,K]ᵀ for MXFP8 operands: e4m3 code tensors A, B
    and their scales packed by mx_pack_scales (operand A resp. B); returns C."""
    import torch
    ok = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    if A.dtype not in ok or B.dtype not in ok:
        raise TypeError("A and B must hold e4m3 bytes (uint8 or float8_e4m3fn)")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A is [M,K] and B is [N,K]")
    for t, rows, name in ((SA_packed, M, "SA_packed"), (SB_packed, N, "SB_packed")):
        need = hkg_mx_packed_scale_bytes(rows, K)
        if need >= 0 and (t.dtype != torch.uint8 or t.numel() < need):
            raise ValueError("%s must be a uint8 tensor of at least %d bytes" % (name, need))
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if tuple(C.shape) != (M, N) or C.dtype != torch.bfloat16:
        raise ValueError("C must be a [M,N] bfloat16 tensor")
    if C_f32 is not None and (tuple(C_f32.shape) != (M, N) or C_f32.dtype != torch.float32):
        raise ValueError("C_f32 must be a [M,N] float32 tensor")
    pA, pB, pC, pF, opts = _operands(A, B, C, C_f32, opts, M, N, K)
    rc = hkg_gemm_mxfp8_ex(M, N, K, pA, pB, _dev_ptr(SA_packed, "SA_packed"),
                           _dev_ptr(SB_packed, "SB_packed"), pC, pF, _stream_handle(stream), opts)
    if rc != HKG_OK:
        raise HkgError(rc, "hkg_gemm_mxfp8_ex")
    return C


def tune_remap(A, B, C=None, launches=10, stream=None):
    """Time the candidate grid orders of C = A·Bᵀ on these GPU tensors (bf16, or
    e4m3 bytes timed with unit scales) and return (opts, ms, tried): the fastest
    as hkg_gemm_opts for gemm_bf16 / gemm_fp8 / gemm_mxfp8, its time per launch,
    and (opts, ms) of every configuration timed (the default launch first).
    C (allocated if None) is overwritten with the product."""
    import torch
    if A.dtype == torch.bfloat16 and B.dtype == torch.bfloat16:
        dtype = 0
    elif A.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)) and \
            B.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        dtype = 1
    else:
        raise TypeError("A and B must both be bfloat16 or both hold e4m3 bytes")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A is [M,K] and B is [N,K]")
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if tuple(C.shape) != (M, N) or C.dtype != torch.bfloat16:
        raise ValueError("C must be a [M,N] bfloat16 tensor")
    best = hkg_gemm_opts()
    rc, ms, tried = hkg_tune_remap(M, N, K, dtype, _dev_ptr(A, "A"), _dev_ptr(B, "B"),
                                   _dev_ptr(C, "C"), launches, best, _stream_handle(stream))
    if rc != HKG_OK:
        raise HkgError(rc, "hkg_tune_remap")
    return best, ms, tried


def remap_tiles_device(Gm, Gn, W, C, stream=None):
    """Device-evaluated grid remap -> int32 GPU tensor [Gm*Gn, 2] of (tile_m, tile_n)."""
    import torch
    out = torch.empty((Gm * Gn, 2), dtype=torch.int32, device="cuda")
    rc = hkg_remap_tiles_device(Gm, Gn, W, C, out.data_ptr(), _stream_handle(stream))
    if rc != HKG_OK:
        raise HkgError(rc, "hkg_remap_tiles_device")
    return out


def probe_xcd(workgroups, full_lds=True, spin_cycles=0, stream=None):
    """Where each workgroup of a launch ran (hkg_probe_xcd) -> int32 GPU tensor
    [workgroups, 2] of (XCC_ID register, HW_ID register)."""
    import torch
    out = torch.empty((workgroups, 2), dtype=torch.int32, device="cuda")
    rc = hkg_probe_xcd(workgroups, int(bool(full_lds)), spin_cycles, out.data_ptr(),
                       _stream_handle(stream))
    if rc != HKG_OK:
        raise HkgError(rc, "hkg_probe_xcd")
    return out
