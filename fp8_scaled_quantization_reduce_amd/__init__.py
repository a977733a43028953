"""fp8_scaled_quantization_reduce_amd -- FP8 scaled quantization and scaled FP8
GEMM for MI355X (gfx950).

This module is a thin ctypes binding over ``libfp8q.so``: the functions carry
the names of the C entry points in ``include/fp8q.h`` and only marshal torch
tensors (device memory) and the current HIP stream into them.  Every step of
the computation runs in the library's HIP kernels; there is no Python or CPU
fallback.  Importing the package fails if the library has not been built
(``python fp8_scaled_quantization_reduce_amd/build.py``).

Tensor conventions: high-precision inputs are ``torch.float32`` or
``torch.bfloat16``; FP8 codes are ``torch.uint8``; scalars (amax, scales) are
one-element ``torch.float32`` tensors on the device.  ``fmt`` is E4M3FN (0) or
E5M2 (1).
"""
from __future__ import annotations

import ctypes
import os

import torch

E4M3FN, E5M2 = 0, 1
F32, BF16 = 0, 1
ALGO_MAX, ALGO_MOST_RECENT = 0, 1
PER_TENSOR, BLOCK_1x128_128x128, BLOCK_1x128_1x128, MXFP8 = 0, 1, 2, 3
OUT_E4M3FN, OUT_E5M2 = 2, 3
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
COLSRC_ORIGINAL, COLSRC_ROWWISE_DEQUANTIZED = 0, 1
OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

# every entry point of include/fp8q.h, with its ctypes argument list
_VP, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "fp8_amax": [_VP, _I32, _I64, _VP, _VP],
    "fp8_quantize_tensor": [_VP, _I32, _I64, _I32, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP],
    "fp8_quantize_tensor_stats": [_VP, _I32, _I64, _I32, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "fp8_dequantize": [_VP, _I32, _I64, _VP, _VP, _VP],
    "fp8_quantize_rowwise_colwise": [_VP, _I32, _I64, _I64, _I32, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "fp8_quantize_block": [_VP, _I32, _I64, _I64, _I32, _I32, _VP, _VP, _VP, _VP, _VP],
    "fp8_quantize_mx": [_VP, _I32, _I64, _I64, _I32, _VP, _VP, _VP, _VP, _VP],
    "fp8_update_scale_delayed": [_VP, _I32, _I32, _I32, _VP, _I64, _I32, _I32, _I32, _VP, _VP, _VP],
    "fp8_quantize_delayed": [_VP, _I32, _I64, _I32, _VP, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _VP, _VP, _VP, _VP,
                             _VP, _VP],
    "fp8_scaled_gemm": [_VP, _I32, _VP, _VP, _I32, _VP, _I64, _I64, _I64, _I32, _VP, _I32, _VP, _VP],
    "fp8_scaled_gemm_fused": [_VP, _I32, _VP, _VP, _I32, _VP, _I64, _I64, _I64, _I32, _VP, _I32, _VP, _I32, _VP, _VP,
                              _VP],
    "fp8_quantize_hybrid": [_VP, _I32, _I64, _I64, _I32, _I32, _I32, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP,
                            _VP, _VP],
    "fp8_cast_stats": [_VP, _I32, _I64, _I32, _VP, _VP, _VP],
    "fp8_quantize_error_feedback": [_VP, _I32, _VP, _I64, _I32, _VP, _VP, _VP, _VP],
    "fp8q_last_error": [],
}


class Fp8qError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("status %d: %s" % (status, message))
        self.status = status


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfp8q.so is not built (%s); build it with "
                          "`python fp8_scaled_quantization_reduce_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name == "fp8q_last_error" else ctypes.c_int
    return lib


lib = _load_library()


def last_error() -> str:
    return lib.fp8q_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise Fp8qError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libfp8q must be contiguous")
    return t.data_ptr()


def _dtype(t) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("high-precision tensors must be float32 or bfloat16, got %s" % t.dtype)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def fp8_amax(x, amax, stream=None):
    """amax[0] = max |x|."""
    _check(lib.fp8_amax(_ptr(x), _dtype(x), x.numel(), _ptr(amax), _stream(stream)))


def fp8_quantize_tensor(x, fmt, q, *, amax_in=None, margin=0, scale_inv_in=None, scale_inv_out=None,
                        scale_out=None, amax_out=None, stream=None):
    """Per-tensor scaled cast; exactly one of amax_in / scale_inv_in."""
    _check(lib.fp8_quantize_tensor(_ptr(x), _dtype(x), x.numel(), fmt, _ptr(amax_in), margin, _ptr(scale_inv_in),
                                   _ptr(q), _ptr(scale_inv_out), _ptr(scale_out), _ptr(amax_out), _stream(stream)))


def fp8_quantize_tensor_stats(x, fmt, q, stats, *, amax_in=None, margin=0, scale_inv_in=None, scale_inv_out=None,
                              scale_out=None, amax_out=None, stream=None):
    """fp8_quantize_tensor that also writes the cast's counts to stats (int64
    [4] on the device: overflows, underflows, NaNs, nonzeros) in the same pass."""
    if stats.dtype not in (torch.int64, torch.uint64) or stats.numel() != 4:
        raise ValueError("stats must be a 4-element 64-bit integer tensor")
    _check(lib.fp8_quantize_tensor_stats(_ptr(x), _dtype(x), x.numel(), fmt, _ptr(amax_in), margin,
                                         _ptr(scale_inv_in), _ptr(q), _ptr(scale_inv_out), _ptr(scale_out),
                                         _ptr(amax_out), _ptr(stats), _stream(stream)))


def fp8_dequantize(q, fmt, scale_inv, y, stream=None):
    """y = value(q) * scale_inv[0]."""
    _check(lib.fp8_dequantize(_ptr(q), fmt, q.numel(), _ptr(scale_inv), _ptr(y), _stream(stream)))


def fp8_quantize_rowwise_colwise(x, fmt, *, q_row=None, q_col=None, amax_in=None, margin=0, scale_inv_in=None,
                                 scale_inv_out=None, scale_out=None, amax_out=None, stream=None):
    """Per-tensor cast of a 2-D tensor to row-major codes and transposed codes."""
    rows, cols = x.shape
    _check(lib.fp8_quantize_rowwise_colwise(_ptr(x), _dtype(x), rows, cols, fmt, _ptr(amax_in), margin,
                                            _ptr(scale_inv_in), _ptr(q_row), _ptr(q_col), _ptr(scale_inv_out),
                                            _ptr(scale_out), _ptr(amax_out), _stream(stream)))


def fp8_quantize_block(x, fmt, block_rows, q_row, s_row, q_col=None, s_col=None, stream=None):
    """Block current scaling (1x128 or 128x128) with optional columnwise copy."""
    rows, cols = x.shape
    _check(lib.fp8_quantize_block(_ptr(x), _dtype(x), rows, cols, fmt, block_rows, _ptr(q_row), _ptr(s_row),
                                  _ptr(q_col), _ptr(s_col), _stream(stream)))


def fp8_quantize_mx(x, fmt, q_row, s_row, q_col=None, s_col=None, stream=None):
    """MXFP8: 1x32 blocks along the rows with E8M0 scale bytes (uint8 tensors),
    optionally the columnwise copy (the same rule on x^T)."""
    rows, cols = x.shape
    _check(lib.fp8_quantize_mx(_ptr(x), _dtype(x), rows, cols, fmt, _ptr(q_row), _ptr(s_row), _ptr(q_col),
                               _ptr(s_col), _stream(stream)))


def fp8_update_scale_delayed(hist, col, new_amax, step, fmt, margin, algo, scale, scale_inv, stream=None):
    """Delayed-scaling update of column `col` of hist [history_len][n_cols]."""
    history_len, n_cols = hist.shape
    _check(lib.fp8_update_scale_delayed(_ptr(hist), history_len, n_cols, col, _ptr(new_amax), step, fmt, margin, algo,
                                        _ptr(scale), _ptr(scale_inv), _stream(stream)))


def fp8_quantize_delayed(x, fmt, hist, col, step, fmt_next, margin, algo, scale, scale_inv, q, q_scale_inv_out=None,
                         amax_out=None, stream=None):
    """One delayed-scaling step: cast with scale_inv[col], then record max|x|
    in column col of hist and update scale/scale_inv for fmt_next."""
    history_len, n_cols = hist.shape
    _check(lib.fp8_quantize_delayed(_ptr(x), _dtype(x), x.numel(), fmt, _ptr(hist), history_len, n_cols, col, step,
                                    fmt_next, margin, algo, _ptr(scale), _ptr(scale_inv), _ptr(q),
                                    _ptr(q_scale_inv_out), _ptr(amax_out), _stream(stream)))


def fp8_scaled_gemm(A, fa, sA, B, fb, sB, mode, C, amax_out=None, stream=None):
    """C = (A*sA)(B*sB)^T, A [M][K], B [N][K] codes, C [M][N] bfloat16 or float32."""
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    _check(lib.fp8_scaled_gemm(_ptr(A), fa, _ptr(sA), _ptr(B), fb, _ptr(sB), M, N, K, mode, _ptr(C), _dtype(C),
                               _ptr(amax_out), _stream(stream)))


def fp8_scaled_gemm_fused(A, fa, sA, B, fb, sB, mode, C, *, bias=None, act=ACT_NONE, out_fmt=None,
                          c_scale_inv=None, amax_out=None, stream=None):
    """C = out(act((A*sA)(B*sB)^T + bias)); C bfloat16 / float32, or uint8
    codes of out_fmt (E4M3FN / E5M2) cast with the dequant scale c_scale_inv."""
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    if C.dtype == torch.uint8:
        if out_fmt not in (E4M3FN, E5M2):
            raise ValueError("a uint8 C needs out_fmt E4M3FN or E5M2")
        c_type = OUT_E4M3FN if out_fmt == E4M3FN else OUT_E5M2
    else:
        c_type = _dtype(C)
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != N):
        raise ValueError("bias must be float32 with N elements")
    _check(lib.fp8_scaled_gemm_fused(_ptr(A), fa, _ptr(sA), _ptr(B), fb, _ptr(sB), M, N, K, mode, _ptr(bias), act,
                                     _ptr(C), c_type, _ptr(c_scale_inv), _ptr(amax_out), _stream(stream)))


def fp8_quantize_hybrid(x, row_fmt, col_fmt, col_source, *, q_row=None, q_col=None, amax_in=None, row_margin=0,
                        col_margin=0, row_scale_inv_in=None, col_scale_inv_in=None, row_scale_inv_out=None,
                        col_scale_inv_out=None, amax_out=None, stream=None):
    """Per-direction per-tensor cast: rowwise codes in row_fmt, columnwise
    (transposed) codes in col_fmt from x or from the dequantized rows."""
    rows, cols = x.shape
    _check(lib.fp8_quantize_hybrid(_ptr(x), _dtype(x), rows, cols, row_fmt, col_fmt, col_source, _ptr(amax_in),
                                   row_margin, col_margin, _ptr(row_scale_inv_in), _ptr(col_scale_inv_in),
                                   _ptr(q_row), _ptr(q_col), _ptr(row_scale_inv_out), _ptr(col_scale_inv_out),
                                   _ptr(amax_out), _stream(stream)))


def fp8_cast_stats(x, fmt, scale_inv, stats, stream=None):
    """stats (int64 [4] on the device) = overflows, underflows, NaNs,
    nonzeros of the cast of x with dequant scale scale_inv."""
    if stats.dtype not in (torch.int64, torch.uint64) or stats.numel() != 4:
        raise ValueError("stats must be a 4-element 64-bit integer tensor")
    _check(lib.fp8_cast_stats(_ptr(x), _dtype(x), x.numel(), fmt, _ptr(scale_inv), _ptr(stats), _stream(stream)))


def fp8_quantize_error_feedback(g, residual, fmt, scale_inv, q, amax_out=None, stream=None):
    """q = cast(g + residual); residual <- (g + residual) - dequant(q), in place."""
    if residual.dtype != torch.float32 or residual.numel() != g.numel():
        raise ValueError("residual must be float32 with g's element count")
    _check(lib.fp8_quantize_error_feedback(_ptr(g), _dtype(g), _ptr(residual), g.numel(), fmt, _ptr(scale_inv),
                                           _ptr(q), _ptr(amax_out), _stream(stream)))
