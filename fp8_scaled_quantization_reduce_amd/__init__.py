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
SUBQ_BLOCK_128x128, SUBQ_BLOCK_1x128, SUBQ_MXFP8, SUBQ_PER_TENSOR = 0, 1, 2, 3
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
    "fp8_quantize_hybrid_blockwise": [_VP, _I32, _I64, _I64, _I32, _I32, _VP, _VP, _I32, _I32, _I32, _VP, _VP,
                                      _VP, _I32, _VP, _VP],
    "fp8_cast_stats": [_VP, _I32, _I64, _I32, _VP, _VP, _VP],
    "fp8_quantize_error_feedback": [_VP, _I32, _VP, _I64, _I32, _VP, _VP, _VP, _VP],
    "fp8q_clock_monitor": [_VP, _VP, _VP],
    "fp8q_set_finish_poll_rounds": [ctypes.c_uint32, _VP],
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


# ------------------------------------------------------- argument checks --
# The C ABI sees only pointers, so it cannot tell a buffer's size, type or
# device; the binding checks them before any call, so that a short output or
# a host tensor raises here instead of reaching a kernel.  Sizes and types are
# checked first and the device last.

def _tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _need(t, name, dtypes, numel=None, at_least=False):
    """t (or None) has one of `dtypes` and exactly `numel` elements (with
    at_least, `numel` or more: an input the kernels read a prefix of)."""
    if t is None:
        return
    _tensor(t, name)
    if t.dtype not in dtypes:
        raise TypeError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if numel is None:
        return
    if at_least and t.numel() < numel:
        raise ValueError("%s must have at least %d elements, got %d" % (name, numel, t.numel()))
    if not at_least and t.numel() != numel:
        raise ValueError("%s must have %d elements, got %d" % (name, numel, t.numel()))


def _need_scalar(t, name):
    _need(t, name, (torch.float32,), 1)


def _ptr(t, name="tensor"):
    """Device address of a contiguous tensor on the current GPU (None -> NULL)."""
    if t is None:
        return None
    _tensor(t, name)
    dev = t.get_device()  # -1 for host tensors
    if dev < 0:
        raise ValueError("%s must be a GPU tensor (device %s)" % (name, t.device))
    if dev != torch.cuda.current_device():
        raise ValueError("%s is on cuda:%d but the current device is cuda:%d" % (name, dev,
                                                                               torch.cuda.current_device()))
    return t.data_ptr()


_HP = (torch.float32, torch.bfloat16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_STATS = (torch.int64, torch.uint64)


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


def _shape2(x, name="x"):
    _need(x, name, _HP)
    if x.dim() != 2:
        raise ValueError("%s must be 2-D, got shape %s" % (name, tuple(x.shape)))
    return x.shape


def fp8_amax(x, amax, stream=None):
    """amax[0] = max |x|."""
    _need(x, "x", _HP)
    _need_scalar(amax, "amax")
    _check(lib.fp8_amax(_ptr(x, "x"), _dtype(x), x.numel(), _ptr(amax, "amax"), _stream(stream)))


def _scalars(**kw):
    for name, t in kw.items():
        if t is not None:
            _need_scalar(t, name)


def fp8_quantize_tensor(x, fmt, q, *, amax_in=None, margin=0, scale_inv_in=None, scale_inv_out=None,
                        scale_out=None, amax_out=None, stream=None):
    """Per-tensor scaled cast; exactly one of amax_in / scale_inv_in."""
    _need(x, "x", _HP)
    _need(q, "q", _U8, x.numel())
    _scalars(amax_in=amax_in, scale_inv_in=scale_inv_in, scale_inv_out=scale_inv_out, scale_out=scale_out,
             amax_out=amax_out)
    _check(lib.fp8_quantize_tensor(_ptr(x, "x"), _dtype(x), x.numel(), fmt, _ptr(amax_in, "amax_in"), margin,
                                   _ptr(scale_inv_in, "scale_inv_in"), _ptr(q, "q"),
                                   _ptr(scale_inv_out, "scale_inv_out"), _ptr(scale_out, "scale_out"),
                                   _ptr(amax_out, "amax_out"), _stream(stream)))


def fp8_quantize_tensor_stats(x, fmt, q, stats, *, amax_in=None, margin=0, scale_inv_in=None, scale_inv_out=None,
                              scale_out=None, amax_out=None, stream=None):
    """fp8_quantize_tensor that also writes the cast's counts to stats (int64
    [4] on the device: overflows, underflows, NaNs, nonzeros) in the same pass."""
    _need(x, "x", _HP)
    _need(q, "q", _U8, x.numel())
    _need(stats, "stats", _STATS, 4)
    _scalars(amax_in=amax_in, scale_inv_in=scale_inv_in, scale_inv_out=scale_inv_out, scale_out=scale_out,
             amax_out=amax_out)
    _check(lib.fp8_quantize_tensor_stats(_ptr(x, "x"), _dtype(x), x.numel(), fmt, _ptr(amax_in, "amax_in"), margin,
                                         _ptr(scale_inv_in, "scale_inv_in"), _ptr(q, "q"),
                                         _ptr(scale_inv_out, "scale_inv_out"), _ptr(scale_out, "scale_out"),
                                         _ptr(amax_out, "amax_out"), _ptr(stats, "stats"), _stream(stream)))


def fp8_dequantize(q, fmt, scale_inv, y, stream=None):
    """y = value(q) * scale_inv[0]."""
    _need(q, "q", _U8)
    _need_scalar(scale_inv, "scale_inv")
    _need(y, "y", _F32, q.numel())
    _check(lib.fp8_dequantize(_ptr(q, "q"), fmt, q.numel(), _ptr(scale_inv, "scale_inv"), _ptr(y, "y"),
                              _stream(stream)))


def fp8_quantize_rowwise_colwise(x, fmt, *, q_row=None, q_col=None, amax_in=None, margin=0, scale_inv_in=None,
                                 scale_inv_out=None, scale_out=None, amax_out=None, stream=None):
    """Per-tensor cast of a 2-D tensor to row-major codes and transposed codes."""
    rows, cols = _shape2(x)
    _need(q_row, "q_row", _U8, rows * cols)
    _need(q_col, "q_col", _U8, rows * cols)
    _scalars(amax_in=amax_in, scale_inv_in=scale_inv_in, scale_inv_out=scale_inv_out, scale_out=scale_out,
             amax_out=amax_out)
    _check(lib.fp8_quantize_rowwise_colwise(_ptr(x, "x"), _dtype(x), rows, cols, fmt, _ptr(amax_in, "amax_in"),
                                            margin, _ptr(scale_inv_in, "scale_inv_in"), _ptr(q_row, "q_row"),
                                            _ptr(q_col, "q_col"), _ptr(scale_inv_out, "scale_inv_out"),
                                            _ptr(scale_out, "scale_out"), _ptr(amax_out, "amax_out"),
                                            _stream(stream)))


def fp8_quantize_block(x, fmt, block_rows, q_row, s_row, q_col=None, s_col=None, stream=None):
    """Block current scaling (1x128 or 128x128) with optional columnwise copy."""
    rows, cols = _shape2(x)
    if block_rows in (1, 128):
        _need(q_row, "q_row", _U8, rows * cols)
        _need(s_row, "s_row", _F32, (rows // block_rows) * (cols // 128))
        _need(q_col, "q_col", _U8, rows * cols)
        _need(s_col, "s_col", _F32, (cols // 128 if block_rows == 128 else cols) * (rows // 128))
    _check(lib.fp8_quantize_block(_ptr(x, "x"), _dtype(x), rows, cols, fmt, block_rows, _ptr(q_row, "q_row"),
                                  _ptr(s_row, "s_row"), _ptr(q_col, "q_col"), _ptr(s_col, "s_col"), _stream(stream)))


def fp8_quantize_mx(x, fmt, q_row, s_row, q_col=None, s_col=None, stream=None):
    """MXFP8: 1x32 blocks along the rows with E8M0 scale bytes (uint8 tensors),
    optionally the columnwise copy (the same rule on x^T)."""
    rows, cols = _shape2(x)
    _need(q_row, "q_row", _U8, rows * cols)
    _need(s_row, "s_row", _U8, rows * (cols // 32))
    _need(q_col, "q_col", _U8, rows * cols)
    _need(s_col, "s_col", _U8, cols * (rows // 32))
    _check(lib.fp8_quantize_mx(_ptr(x, "x"), _dtype(x), rows, cols, fmt, _ptr(q_row, "q_row"), _ptr(s_row, "s_row"),
                               _ptr(q_col, "q_col"), _ptr(s_col, "s_col"), _stream(stream)))


def _delayed_state(hist, new_amax, scale, scale_inv):
    _need(hist, "hist", _F32)
    if hist.dim() != 2:
        raise ValueError("hist must be [history_len][n_cols], got shape %s" % (tuple(hist.shape),))
    n_cols = hist.shape[1]
    if new_amax is not None:
        _need_scalar(new_amax, "new_amax")
    _need(scale, "scale", _F32, n_cols)
    _need(scale_inv, "scale_inv", _F32, n_cols)
    return hist.shape


def fp8_update_scale_delayed(hist, col, new_amax, step, fmt, margin, algo, scale, scale_inv, stream=None):
    """Delayed-scaling update of column `col` of hist [history_len][n_cols]."""
    if new_amax is None:
        raise ValueError("new_amax is required")
    history_len, n_cols = _delayed_state(hist, new_amax, scale, scale_inv)
    _check(lib.fp8_update_scale_delayed(_ptr(hist, "hist"), history_len, n_cols, col, _ptr(new_amax, "new_amax"),
                                        step, fmt, margin, algo, _ptr(scale, "scale"), _ptr(scale_inv, "scale_inv"),
                                        _stream(stream)))


def fp8_quantize_delayed(x, fmt, hist, col, step, fmt_next, margin, algo, scale, scale_inv, q, q_scale_inv_out=None,
                         amax_out=None, stream=None):
    """One delayed-scaling step: cast with scale_inv[col], then record max|x|
    in column col of hist and update scale/scale_inv for fmt_next."""
    _need(x, "x", _HP)
    history_len, n_cols = _delayed_state(hist, None, scale, scale_inv)
    _need(q, "q", _U8, x.numel())
    _scalars(q_scale_inv_out=q_scale_inv_out, amax_out=amax_out)
    _check(lib.fp8_quantize_delayed(_ptr(x, "x"), _dtype(x), x.numel(), fmt, _ptr(hist, "hist"), history_len, n_cols,
                                    col, step, fmt_next, margin, algo, _ptr(scale, "scale"),
                                    _ptr(scale_inv, "scale_inv"), _ptr(q, "q"),
                                    _ptr(q_scale_inv_out, "q_scale_inv_out"), _ptr(amax_out, "amax_out"),
                                    _stream(stream)))


def _gemm_operands(A, sA, B, sB, mode, C):
    """Shapes of C = A B^T and the scale buffers each mode reads."""
    _need(A, "A", _U8)
    _need(B, "B", _U8)
    if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
        raise ValueError("A, B and C must be 2-D")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    # scale buffers are read, never written: a longer one is harmless (a
    # K = 0 product reads none but still needs a buffer)
    if mode == PER_TENSOR:
        _need(sA, "sA", _F32, 1)
        _need(sB, "sB", _F32, 1)
    elif mode == BLOCK_1x128_128x128:
        _need(sA, "sA", _F32, max(1, M * (K // 128)), at_least=True)
        _need(sB, "sB", _F32, max(1, (N // 128) * (K // 128)), at_least=True)
    elif mode == BLOCK_1x128_1x128:
        _need(sA, "sA", _F32, max(1, M * (K // 128)), at_least=True)
        _need(sB, "sB", _F32, max(1, N * (K // 128)), at_least=True)
    elif mode == MXFP8:
        _need(sA, "sA", _U8, max(1, M * (K // 32)), at_least=True)
        _need(sB, "sB", _U8, max(1, N * (K // 32)), at_least=True)
    if sA is None or sB is None:
        raise ValueError("sA and sB are required")
    return M, N, K


def fp8_scaled_gemm(A, fa, sA, B, fb, sB, mode, C, amax_out=None, stream=None):
    """C = (A*sA)(B*sB)^T, A [M][K], B [N][K] codes, C [M][N] bfloat16 or float32."""
    _need(C, "C", _HP)
    M, N, K = _gemm_operands(A, sA, B, sB, mode, C)
    _scalars(amax_out=amax_out)
    _check(lib.fp8_scaled_gemm(_ptr(A, "A"), fa, _ptr(sA, "sA"), _ptr(B, "B"), fb, _ptr(sB, "sB"), M, N, K, mode,
                               _ptr(C, "C"), _dtype(C), _ptr(amax_out, "amax_out"), _stream(stream)))


def fp8_scaled_gemm_fused(A, fa, sA, B, fb, sB, mode, C, *, bias=None, act=ACT_NONE, out_fmt=None,
                          c_scale_inv=None, amax_out=None, stream=None):
    """C = out(act((A*sA)(B*sB)^T + bias)); C bfloat16 / float32, or uint8
    codes of out_fmt (E4M3FN / E5M2) cast with the dequant scale c_scale_inv."""
    _need(C, "C", (torch.float32, torch.bfloat16, torch.uint8))
    M, N, K = _gemm_operands(A, sA, B, sB, mode, C)
    if C.dtype == torch.uint8:
        if out_fmt not in (E4M3FN, E5M2):
            raise ValueError("a uint8 C needs out_fmt E4M3FN or E5M2")
        c_type = OUT_E4M3FN if out_fmt == E4M3FN else OUT_E5M2
        if c_scale_inv is None:
            raise ValueError("an FP8 output needs c_scale_inv")
    else:
        c_type = _dtype(C)
    _need(bias, "bias", _F32, N)
    _scalars(c_scale_inv=c_scale_inv, amax_out=amax_out)
    _check(lib.fp8_scaled_gemm_fused(_ptr(A, "A"), fa, _ptr(sA, "sA"), _ptr(B, "B"), fb, _ptr(sB, "sB"), M, N, K,
                                     mode, _ptr(bias, "bias"), act, _ptr(C, "C"), c_type,
                                     _ptr(c_scale_inv, "c_scale_inv"), _ptr(amax_out, "amax_out"), _stream(stream)))


def fp8_quantize_hybrid(x, row_fmt, col_fmt, col_source, *, q_row=None, q_col=None, amax_in=None, row_margin=0,
                        col_margin=0, row_scale_inv_in=None, col_scale_inv_in=None, row_scale_inv_out=None,
                        col_scale_inv_out=None, amax_out=None, stream=None):
    """Per-direction per-tensor cast: rowwise codes in row_fmt, columnwise
    (transposed) codes in col_fmt from x or from the dequantized rows."""
    rows, cols = _shape2(x)
    _need(q_row, "q_row", _U8, rows * cols)
    _need(q_col, "q_col", _U8, rows * cols)
    _scalars(amax_in=amax_in, row_scale_inv_in=row_scale_inv_in, col_scale_inv_in=col_scale_inv_in,
             row_scale_inv_out=row_scale_inv_out, col_scale_inv_out=col_scale_inv_out, amax_out=amax_out)
    _check(lib.fp8_quantize_hybrid(_ptr(x, "x"), _dtype(x), rows, cols, row_fmt, col_fmt, col_source,
                                   _ptr(amax_in, "amax_in"), row_margin, col_margin,
                                   _ptr(row_scale_inv_in, "row_scale_inv_in"),
                                   _ptr(col_scale_inv_in, "col_scale_inv_in"), _ptr(q_row, "q_row"),
                                   _ptr(q_col, "q_col"), _ptr(row_scale_inv_out, "row_scale_inv_out"),
                                   _ptr(col_scale_inv_out, "col_scale_inv_out"), _ptr(amax_out, "amax_out"),
                                   _stream(stream)))


def _subq_scales(recipe, rows, cols):
    """(dtype, element count) of the scale buffer of one direction's copy of a
    [rows][cols] tensor under a sub-quantizer."""
    if recipe == SUBQ_PER_TENSOR:
        return _F32, 1
    if recipe == SUBQ_BLOCK_128x128:
        return _F32, (rows // 128) * (cols // 128)
    if recipe == SUBQ_BLOCK_1x128:
        return _F32, rows * (cols // 128)
    return _U8, rows * (cols // 32)


def fp8_quantize_hybrid_blockwise(x, row_recipe, row_fmt, col_recipe, col_fmt, *, col_source=COLSRC_ORIGINAL,
                                  q_row=None, s_row=None, q_col=None, s_col=None, amax_in=None, margin=0,
                                  scale_inv_in=None, stream=None):
    """Per-direction quantization with block, MXFP8 or (in one direction)
    per-tensor sub-quantizers: rowwise copy by row_recipe in row_fmt (codes
    [rows][cols]), columnwise copy by col_recipe in col_fmt applied to x^T or
    to the dequantized rows (codes [cols][rows]); scales float32 (blocks; one
    float for a per-tensor direction, which takes amax_in or scale_inv_in) or
    uint8 (MXFP8)."""
    rows, cols = _shape2(x)
    recipes = (SUBQ_BLOCK_128x128, SUBQ_BLOCK_1x128, SUBQ_MXFP8, SUBQ_PER_TENSOR)
    if row_recipe in recipes:
        _need(q_row, "q_row", _U8, rows * cols)
        _need(s_row, "s_row", *_subq_scales(row_recipe, rows, cols))
    if col_recipe in recipes:
        _need(q_col, "q_col", _U8, rows * cols)
        _need(s_col, "s_col", *_subq_scales(col_recipe, cols, rows))
    _scalars(amax_in=amax_in, scale_inv_in=scale_inv_in)
    _check(lib.fp8_quantize_hybrid_blockwise(_ptr(x, "x"), _dtype(x), rows, cols, row_recipe, row_fmt,
                                             _ptr(q_row, "q_row"), _ptr(s_row, "s_row"), col_recipe, col_fmt,
                                             col_source, _ptr(q_col, "q_col"), _ptr(s_col, "s_col"),
                                             _ptr(amax_in, "amax_in"), margin, _ptr(scale_inv_in, "scale_inv_in"),
                                             _stream(stream)))


def fp8_cast_stats(x, fmt, scale_inv, stats, stream=None):
    """stats (int64 [4] on the device) = overflows, underflows, NaNs,
    nonzeros of the cast of x with dequant scale scale_inv."""
    _need(x, "x", _HP)
    _need_scalar(scale_inv, "scale_inv")
    _need(stats, "stats", _STATS, 4)
    _check(lib.fp8_cast_stats(_ptr(x, "x"), _dtype(x), x.numel(), fmt, _ptr(scale_inv, "scale_inv"),
                              _ptr(stats, "stats"), _stream(stream)))


def fp8_quantize_error_feedback(g, residual, fmt, scale_inv, q, amax_out=None, stream=None):
    """q = cast(g + residual); residual <- (g + residual) - dequant(q), in place."""
    _need(g, "g", _HP)
    _need(residual, "residual", _F32, g.numel())
    _need(q, "q", _U8, g.numel())
    _need_scalar(scale_inv, "scale_inv")
    _scalars(amax_out=amax_out)
    _check(lib.fp8_quantize_error_feedback(_ptr(g, "g"), _dtype(g), _ptr(residual, "residual"), g.numel(), fmt,
                                           _ptr(scale_inv, "scale_inv"), _ptr(q, "q"), _ptr(amax_out, "amax_out"),
                                           _stream(stream)))


CLOCK_BLOCKS = 8
CLOCK_MONITOR_SECONDS = 2


def fp8q_clock_monitor(out, stop, stream=None):
    """Enqueue the clock monitor (a measurement aid): out (int64 [25] on the
    device) receives, per block b, the XCD id, the shader-clock cycles and
    the constant-rate ticks from the kernel's start until stop (int32 [1] on
    the device) becomes nonzero; out[24] = the constant rate in kHz."""
    _need(out, "out", _STATS, 3 * CLOCK_BLOCKS + 1)
    _need(stop, "stop", (torch.int32,), 1)
    _check(lib.fp8q_clock_monitor(_ptr(out, "out"), _ptr(stop, "stop"), _stream(stream)))


POLL_ROUNDS_DEFAULT = 0xFFFFFFFF


def fp8q_set_finish_poll_rounds(rounds):
    """Set the bound on a finishing block's polling rounds for later calls
    (a failure-handling knob; 0 makes every finishing block give up at once,
    POLL_ROUNDS_DEFAULT restores the default) and return the bound that was
    in force."""
    if not 0 <= int(rounds) <= 0xFFFFFFFF:
        raise ValueError("rounds must fit in 32 bits")
    prev = ctypes.c_uint32(0)
    _check(lib.fp8q_set_finish_poll_rounds(ctypes.c_uint32(int(rounds)), ctypes.byref(prev)))
    return prev.value


def clock_mhz(sample):
    """{xcd: MHz} from a host copy of a clock-monitor output (an XCD measured
    by several blocks keeps their mean); None for a monitor that ran into its
    time limit instead of seeing stop."""
    khz = int(sample[3 * CLOCK_BLOCKS])
    if khz <= 0:
        return None
    acc = {}
    for b in range(CLOCK_BLOCKS):
        cycles, ticks = int(sample[3 * b + 1]), int(sample[3 * b + 2])
        if ticks >= khz * 1000 * CLOCK_MONITOR_SECONDS or cycles <= 0 or ticks <= 0:
            return None
        acc.setdefault(int(sample[3 * b]), []).append(cycles / (ticks / (khz * 1e3)) / 1e6)
    return {x: sum(v) / len(v) for x, v in sorted(acc.items())}
