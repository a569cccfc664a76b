"""ctypes binding of libfp8mi (include/fp8mi.h): argument marshalling only.

Every function here takes torch tensors that already live on the GPU, turns
them into raw device pointers, sizes and enum codes, and calls the C entry
point of the same name on the current HIP stream (or the stream given).  No
arithmetic of the FP8 path happens in Python: amax, scaling, casting and the
GEMMs all run in the HIP kernels of libfp8mi.so.  If the library is missing
or cannot be loaded, every call raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["E4M3", "E5M2", "F32", "BF16", "ACCUM_EXACT", "ACCUM_MFMA_FP8", "QUANTIZE_WORKSPACE_BYTES", "Fp8Error", "load_library", "library_path",
           "status_string", "version", "fp8_quantize", "fp8_amax_update", "fp8_gemm",
           "fp8_quantize_blockwise", "fp8_grouped_gemm", "fp8_gemm_requant", "fp8_shared_scale", "fp8_dequant_sum",
           "fp8_quantize_mx", "fp8_gemm_mx", "mx_scale_ld", "mx_scale_pos", "fp8_quantize_update",
           "fp8_quantize_update_noalloc", "EXPORTED_SYMBOLS"]

E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
ACCUM_EXACT, ACCUM_MFMA_FP8 = 0, 1
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}
ACCUMS = {"exact": ACCUM_EXACT, "mfma_fp8": ACCUM_MFMA_FP8, ACCUM_EXACT: ACCUM_EXACT,
          ACCUM_MFMA_FP8: ACCUM_MFMA_FP8}

EXPORTED_SYMBOLS = ("fp8mi_status_string", "fp8mi_version", "fp8_quantize", "fp8_amax_update",
                    "fp8_gemm", "fp8_quantize_blockwise", "fp8_grouped_gemm", "fp8_gemm_requant",
                    "fp8_shared_scale", "fp8_dequant_sum", "fp8_quantize_mx", "fp8_gemm_mx",
                    "fp8_quantize_update", "fp8_quantize_update_noalloc")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.environ.get("FP8MI_LIBRARY", os.path.join(_HERE, "lib", "libfp8mi.so"))


# Workspace size that lets a cast grid cover the device (FP8MI_QUANTIZE_WORKSPACE_BYTES).
QUANTIZE_WORKSPACE_BYTES = 65536


class Fp8Error(RuntimeError):
    """A libfp8mi entry point returned a non-zero status."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: status {status} ({status_string(status)})")


def load_library():
    """Load libfp8mi.so once and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libfp8mi.so is not built ({path} missing); run __graft_entry__.build() "
                           "or python -m fp8_precision_numerics_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.fp8mi_status_string.argtypes = [ctypes.c_int]
    lib.fp8mi_status_string.restype = ctypes.c_char_p
    lib.fp8mi_version.argtypes = []
    lib.fp8mi_version.restype = ctypes.c_int
    lib.fp8_quantize.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                 vp]
    lib.fp8_quantize.restype = ctypes.c_int
    lib.fp8_quantize_update.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                        vp, i32, vp, vp, vp, vp, vp, vp]
    lib.fp8_quantize_update.restype = ctypes.c_int
    lib.fp8_quantize_update_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, i32,
                                                vp, vp, vp, vp, vp, vp]
    lib.fp8_quantize_update_noalloc.restype = ctypes.c_int
    lib.fp8_amax_update.argtypes = [vp, i32, vp, vp, ctypes.c_int, vp, vp, vp, vp]
    lib.fp8_amax_update.restype = ctypes.c_int
    lib.fp8_gemm.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, vp, vp,
                             ctypes.c_int, ctypes.c_int, vp]
    lib.fp8_gemm.restype = ctypes.c_int
    lib.fp8_quantize_blockwise.argtypes = [vp, ctypes.c_int, i64, i64, i32, ctypes.c_int, vp, vp, vp]
    lib.fp8_quantize_blockwise.restype = ctypes.c_int
    lib.fp8_grouped_gemm.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.fp8_grouped_gemm.restype = ctypes.c_int
    lib.fp8_gemm_requant.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64, i64, vp, vp, ctypes.c_int, vp,
                                     vp, vp, vp, ctypes.c_int, vp]
    lib.fp8_gemm_requant.restype = ctypes.c_int
    lib.fp8_shared_scale.argtypes = [vp, i32, ctypes.c_int, vp, vp, vp]
    lib.fp8_shared_scale.restype = ctypes.c_int
    lib.fp8_dequant_sum.argtypes = [vp, i32, i64, i64, ctypes.c_int, vp, vp, ctypes.c_int, vp]
    lib.fp8_dequant_sum.restype = ctypes.c_int
    lib.fp8_quantize_mx.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.c_int, vp, vp, vp]
    lib.fp8_quantize_mx.restype = ctypes.c_int
    lib.fp8_gemm_mx.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i64, i64, i64, vp, ctypes.c_int,
                                ctypes.c_int, vp]
    lib.fp8_gemm_mx.restype = ctypes.c_int
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fp8mi_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().fp8mi_version())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _xtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"input dtype must be float32 or bfloat16, got {x.dtype}")


def _accum(a) -> int:
    try:
        return ACCUMS[a]
    except KeyError:
        raise ValueError(f"unknown accumulation mode {a!r}") from None


def _fmt(f) -> int:
    try:
        return FORMATS[f]
    except KeyError:
        raise ValueError(f"unknown FP8 format {f!r}") from None


def _check(t, name, dtype=None, numel=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _rows_cols(x: torch.Tensor):
    if x.dim() == 0:
        return 1, 1
    cols = x.shape[-1]
    return (x.numel() // cols if cols else 0), cols


def _call(name, status):
    if status != 0:
        raise Fp8Error(name, status)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def fp8_quantize(x, fmt, scale=None, q=None, q_t=None, amax=None, sat=None, workspace=None, stream=None) -> None:
    """Fused amax + scaled saturating cast of x ([rows x cols], fp32 or bf16).

    q: uint8 [rows x cols] or None; q_t: uint8 [cols x rows] or None;
    scale: fp32[1] device scale; amax: fp32[1] (overwritten); sat: int64[1]
    (overwritten with the saturated-element count); workspace: optional uint8
    device scratch (QUANTIZE_WORKSPACE_BYTES lets the grid cover the device) for
    the per-workgroup partials of amax and the count.
    """
    lib = load_library()
    _check(x, "x", (torch.float32, torch.bfloat16))
    rows, cols = _rows_cols(x)
    dev = x.device
    _check(scale, "scale", torch.float32, 1, dev)
    _check(q, "q", torch.uint8, rows * cols, dev)
    _check(q_t, "q_t", torch.uint8, rows * cols, dev)
    _check(amax, "amax", torch.float32, 1, dev)
    _check(sat, "sat", torch.int64, 1, dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    with torch.cuda.device(dev):
        _call("fp8_quantize", lib.fp8_quantize(_p(x), _xtype(x), rows, cols, _fmt(fmt), _p(scale), _p(q),
                                               _p(q_t), _p(amax), _p(sat), _p(workspace), ws_bytes,
                                               _stream(stream)))


def fp8_quantize_update(x, fmt, history, head, scale, scale_inv, amax, q=None, q_t=None, sat=None, status=None,
                        workspace=None, scale_inv_used=None, stream=None) -> None:
    """fp8_quantize (with the scale as it is) then fp8_amax_update (which refreshes it), in one call;
    scale_inv_used receives the inverse of the scale the cast used (what a GEMM on q needs)."""
    lib = load_library()
    dev = x.device
    _check(x, "x", (torch.float32, torch.bfloat16), None, dev)
    rows, cols = _rows_cols(x)
    _check(q, "q", torch.uint8, rows * cols, dev)
    _check(q_t, "q_t", torch.uint8, rows * cols, dev)
    _check(history, "history", torch.float32, None, dev)
    _check(head, "head", torch.int32, 1, dev)
    _check(scale, "scale", torch.float32, 1, dev)
    _check(scale_inv, "scale_inv", torch.float32, 1, dev)
    _check(amax, "amax", torch.float32, 1, dev)
    _check(sat, "sat", torch.int64, 1, dev)
    _check(status, "status", torch.int32, 1, dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    _check(scale_inv_used, "scale_inv_used", torch.float32, 1, dev)
    xtype = F32 if x.dtype == torch.float32 else BF16
    with torch.cuda.device(dev):
        _call("fp8_quantize_update", lib.fp8_quantize_update(
            _p(x), xtype, rows, cols, _fmt(fmt), _p(q), _p(q_t), _p(amax), _p(sat), _p(workspace),
            workspace.numel() if workspace is not None else 0, _p(history), history.numel(), _p(head), _p(scale),
            _p(scale_inv), _p(status), _p(scale_inv_used), _stream(stream)))


def fp8_quantize_update_noalloc(x, fmt, history, head, scale, scale_inv, amax, q=None, q_t=None, sat=None,
                                status=None, scale_inv_used=None, stream=None) -> None:
    """fp8_quantize_update with the library's own per-GPU scratch instead of a workspace: allocates nothing.
    Calls that may overlap on one GPU must not be issued (they share the scratch)."""
    lib = load_library()
    dev = x.device
    _check(x, "x", (torch.float32, torch.bfloat16), None, dev)
    rows, cols = _rows_cols(x)
    _check(q, "q", torch.uint8, rows * cols, dev)
    _check(q_t, "q_t", torch.uint8, rows * cols, dev)
    _check(history, "history", torch.float32, None, dev)
    _check(head, "head", torch.int32, 1, dev)
    _check(scale, "scale", torch.float32, 1, dev)
    _check(scale_inv, "scale_inv", torch.float32, 1, dev)
    _check(amax, "amax", torch.float32, 1, dev)
    _check(sat, "sat", torch.int64, 1, dev)
    _check(status, "status", torch.int32, 1, dev)
    _check(scale_inv_used, "scale_inv_used", torch.float32, 1, dev)
    xtype = F32 if x.dtype == torch.float32 else BF16
    with torch.cuda.device(dev):
        _call("fp8_quantize_update_noalloc", lib.fp8_quantize_update_noalloc(
            _p(x), xtype, rows, cols, _fmt(fmt), _p(q), _p(q_t), _p(amax), _p(sat), _p(history), history.numel(),
            _p(head), _p(scale), _p(scale_inv), _p(status), _p(scale_inv_used), _stream(stream)))


def fp8_amax_update(history, head, amax, fmt, scale, scale_inv, status=None, stream=None) -> None:
    """Delayed-scaling step: push amax into the ring, recompute scale / scale_inv."""
    lib = load_library()
    dev = history.device
    _check(history, "history", torch.float32, None, dev)
    _check(head, "head", torch.int32, 1, dev)
    _check(amax, "amax", torch.float32, 1, dev)
    _check(scale, "scale", torch.float32, 1, dev)
    _check(scale_inv, "scale_inv", torch.float32, 1, dev)
    _check(status, "status", torch.int32, 1, dev)
    with torch.cuda.device(dev):
        _call("fp8_amax_update", lib.fp8_amax_update(_p(history), history.numel(), _p(head), _p(amax),
                                                     _fmt(fmt), _p(scale), _p(scale_inv), _p(status),
                                                     _stream(stream)))


def fp8_gemm(a, fa, b, fb, sinv_a, sinv_b, c, accum="exact", b_trans=False, stream=None) -> None:
    """C[M x N] = (A[M x K] · B_kn) · sinv_a · sinv_b with FP8 codes A, B, where
    B_kn = b.T for b [N x K] (b_trans False) or b itself for b [K x N] (b_trans True).

    accum: "exact" (every product exact, fp32 sums) or "mfma_fp8" (native FP8
    matrix cores; see include/fp8mi.h for their arithmetic).
    """
    lib = load_library()
    dev = a.device
    _check(a, "a", torch.uint8, None, dev)
    _check(b, "b", torch.uint8, None, dev)
    _check(sinv_a, "sinv_a", torch.float32, 1, dev)
    _check(sinv_b, "sinv_b", torch.float32, 1, dev)
    _check(c, "c", (torch.float32, torch.bfloat16), None, dev)
    M, K = a.shape
    K2, N = b.shape if b_trans else (b.shape[1], b.shape[0])
    if K2 != K or tuple(c.shape) != (M, N):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)} (b_trans={bool(b_trans)}), "
                         f"c {tuple(c.shape)}")
    ctype = F32 if c.dtype == torch.float32 else BF16
    with torch.cuda.device(dev):
        _call("fp8_gemm", lib.fp8_gemm(_p(a), _fmt(fa), _p(b), _fmt(fb), 1 if b_trans else 0, M, N, K, _p(sinv_a),
                                       _p(sinv_b), _p(c), ctype, _accum(accum), _stream(stream)))


def fp8_gemm_requant(a, fa, b, fb, sinv_a, sinv_b, out_fmt, out_scale, cq, amax=None, sat=None, accum="exact",
                     stream=None) -> None:
    """Cq[M x N] = FP8 codes (out_fmt) of fp32((A · Bᵀ) · sinv_a · sinv_b) × out_scale,
    with the amax of the unscaled result and the saturation count (both optional)."""
    lib = load_library()
    dev = a.device
    _check(a, "a", torch.uint8, None, dev)
    _check(b, "b", torch.uint8, None, dev)
    _check(sinv_a, "sinv_a", torch.float32, 1, dev)
    _check(sinv_b, "sinv_b", torch.float32, 1, dev)
    _check(out_scale, "out_scale", torch.float32, 1, dev)
    _check(cq, "cq", torch.uint8, None, dev)
    _check(amax, "amax", torch.float32, 1, dev)
    _check(sat, "sat", torch.int64, 1, dev)
    M, K = a.shape
    N, K2 = b.shape
    if K2 != K or tuple(cq.shape) != (M, N):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, cq {tuple(cq.shape)}")
    with torch.cuda.device(dev):
        _call("fp8_gemm_requant", lib.fp8_gemm_requant(_p(a), _fmt(fa), _p(b), _fmt(fb), M, N, K, _p(sinv_a),
                                                       _p(sinv_b), _fmt(out_fmt), _p(out_scale), _p(cq), _p(amax),
                                                       _p(sat), _accum(accum), _stream(stream)))


def fp8_shared_scale(amaxes, fmt, scale, scale_inv, stream=None) -> None:
    """scale = MAX / max(amaxes) (and its inverse), shared by the ranks of an FP8 all-reduce."""
    lib = load_library()
    dev = amaxes.device
    _check(amaxes, "amaxes", torch.float32, None, dev)
    _check(scale, "scale", torch.float32, 1, dev)
    _check(scale_inv, "scale_inv", torch.float32, 1, dev)
    with torch.cuda.device(dev):
        _call("fp8_shared_scale", lib.fp8_shared_scale(_p(amaxes), amaxes.numel(), _fmt(fmt), _p(scale),
                                                       _p(scale_inv), _stream(stream)))


def fp8_dequant_sum(q, fmt, scale_inv, out, stream=None) -> None:
    """out[i] = (sum over rows r of q, in row order, of dec(q[r, i])) * scale_inv, fp32 sums.

    q: [R x n] uint8 payloads (rows may be a strided view with a 16-byte multiple row stride)."""
    lib = load_library()
    dev = q.device
    if not q.is_cuda or q.dim() != 2 or q.dtype != torch.uint8 or q.stride(1) != 1:
        raise ValueError("q must be a [R x n] uint8 GPU tensor with contiguous rows")
    _check(scale_inv, "scale_inv", torch.float32, 1, dev)
    _check(out, "out", (torch.float32, torch.bfloat16), None, dev)
    R, n = q.shape
    if out.numel() != n:
        raise ValueError(f"out must have {n} elements")
    otype = F32 if out.dtype == torch.float32 else BF16
    with torch.cuda.device(dev):
        # an empty payload addresses nothing: torch reports row stride 1 for [R x 0]
        stride = q.stride(0) if n else 0
        _call("fp8_dequant_sum", lib.fp8_dequant_sum(_p(q), R, n, stride, _fmt(fmt), _p(scale_inv), _p(out),
                                                     otype, _stream(stream)))


def mx_scale_ld(rows: int) -> int:
    """Leading dimension of MXFP8 scale matrices: rows rounded up to 64."""
    return (rows + 63) // 64 * 64


def mx_scale_pos(r):
    """Position of row r inside a K block of an MXFP8 scale matrix (rows permuted within groups of 64)."""
    return (r & ~63) | ((r & 15) << 2) | ((r >> 4) & 3)


def fp8_quantize_mx(x, fmt, q, scales, stream=None) -> None:
    """MXFP8: codes q [rows x cols] and one exponent code per 32 values of a row, stored K-block major:
    scales [cols/32 x mx_scale_ld(rows)], block b of row r at scales[b, mx_scale_pos(r)]."""
    lib = load_library()
    dev = x.device
    _check(x, "x", (torch.float32, torch.bfloat16), None, dev)
    rows, cols = _rows_cols(x)
    _check(q, "q", torch.uint8, rows * cols, dev)
    _check(scales, "scales", torch.uint8, (cols // 32) * mx_scale_ld(rows), dev)
    xtype = F32 if x.dtype == torch.float32 else BF16
    with torch.cuda.device(dev):
        _call("fp8_quantize_mx", lib.fp8_quantize_mx(_p(x), xtype, rows, cols, _fmt(fmt), _p(q), _p(scales),
                                                     _stream(stream)))


def fp8_gemm_mx(a, fa, sa, b, fb, sb, c, accum="exact", stream=None) -> None:
    """C[M x N] = sum_k (dec(a) 2^(sa - 127)) (dec(b) 2^(sb - 127)) on MXFP8 operands a [M x K], b [N x K];
    sa [K/32 x mx_scale_ld(M)], sb [K/32 x mx_scale_ld(N)] as fp8_quantize_mx writes them.
    accum: "exact" (exact products, fp32 sums; rows whose block scales span more than 47 give NaN) or
    "mfma_fp8" (the block-scaled FP8 matrix cores)."""
    lib = load_library()
    dev = a.device
    _check(a, "a", torch.uint8, None, dev)
    _check(b, "b", torch.uint8, None, dev)
    M, K = a.shape
    N, K2 = b.shape
    _check(sa, "sa", torch.uint8, (K // 32) * mx_scale_ld(M), dev)
    _check(sb, "sb", torch.uint8, (K // 32) * mx_scale_ld(N), dev)
    _check(c, "c", (torch.float32, torch.bfloat16), None, dev)
    if K2 != K or tuple(c.shape) != (M, N):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, c {tuple(c.shape)}")
    ctype = F32 if c.dtype == torch.float32 else BF16
    with torch.cuda.device(dev):
        _call("fp8_gemm_mx", lib.fp8_gemm_mx(_p(a), _fmt(fa), _p(sa), _p(b), _fmt(fb), _p(sb), M, N, K, _p(c), ctype,
                                             _accum(accum), _stream(stream)))


def fp8_quantize_blockwise(x, block_rows, fmt, q, scale_inv, stream=None) -> None:
    """Per-block current scaling of x [rows x cols] with block_rows x 128 blocks."""
    lib = load_library()
    _check(x, "x", (torch.float32, torch.bfloat16))
    rows, cols = _rows_cols(x)
    dev = x.device
    _check(q, "q", torch.uint8, rows * cols, dev)
    nbr = (rows + block_rows - 1) // block_rows if block_rows > 0 else 0
    _check(scale_inv, "scale_inv", torch.float32, nbr * ((cols + 127) // 128), dev)
    with torch.cuda.device(dev):
        _call("fp8_quantize_blockwise", lib.fp8_quantize_blockwise(_p(x), _xtype(x), rows, cols, int(block_rows),
                                                                   _fmt(fmt), _p(q), _p(scale_inv),
                                                                   _stream(stream)))


def fp8_grouped_gemm(a, sinv_a, b, sinv_b, m_offsets, c, accum="exact", stream=None) -> None:
    """Grouped fine-grained GEMM: a [total_m x K], b [G x N x K], m_offsets int32 [G+1]."""
    lib = load_library()
    dev = a.device
    _check(a, "a", torch.uint8, None, dev)
    _check(b, "b", torch.uint8, None, dev)
    _check(sinv_a, "sinv_a", torch.float32, None, dev)
    _check(sinv_b, "sinv_b", torch.float32, None, dev)
    _check(m_offsets, "m_offsets", torch.int32, None, dev)
    _check(c, "c", (torch.float32, torch.bfloat16), None, dev)
    total_m, K = a.shape
    G, N, K2 = b.shape
    if K2 != K or tuple(c.shape) != (total_m, N) or m_offsets.numel() != G + 1:
        raise ValueError("shape mismatch in fp8_grouped_gemm")
    ctype = F32 if c.dtype == torch.float32 else BF16
    with torch.cuda.device(dev):
        _call("fp8_grouped_gemm", lib.fp8_grouped_gemm(_p(a), _p(sinv_a), _p(b), _p(sinv_b), _p(m_offsets), G,
                                                       total_m, N, K, _p(c), ctype, _accum(accum),
                                                       _stream(stream)))
