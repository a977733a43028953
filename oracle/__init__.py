"""CPU oracle for FP8 scaled quantization and the scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  The product path (the HIP library and its Python
binding) never imports, links or runs anything in this package; only the tests,
the smoke check and the benchmark's CPU-baseline leg do.  It shares no code
with the HIP path.

The element-wise parts live in plain C (``fp8_oracle.c``, built with gcc,
OpenMP over elements); this module marshals numpy arrays into it and adds the
GEMM reference, which uses numpy's float64 matmul as its one library step.

Conventions: bf16 tensors are numpy ``uint16`` arrays of bf16 bit patterns;
FP8 codes are ``uint8``; scales are ``float32`` scalars.  ``fmt`` is 0 for
E4M3FN, 1 for E5M2.

Pages cited (title, section): "Megatron FP8" (sections 1-28),
"[Pytorch][Common] Hybrid quantization #2817" (TransformerEngine PR),
"Low Precision Training and Rollout" (vime documentation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

E4M3FN, E5M2 = 0, 1
F32, BF16 = 0, 1
ALGO_MAX, ALGO_MOST_RECENT = 0, 1
PER_TENSOR, BLOCK_1x128_128x128, BLOCK_1x128_1x128, MXFP8 = 0, 1, 2, 3
SUBQ_BLOCK_128x128, SUBQ_BLOCK_1x128, SUBQ_MXFP8, SUBQ_PER_TENSOR = 0, 1, 2, 3
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
            vp, fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)
            lib.orc_decode.restype = ctypes.c_double
            lib.orc_decode.argtypes = [i32, i32]
            lib.orc_fmax.restype = ctypes.c_double
            lib.orc_fmax.argtypes = [i32]
            lib.orc_max_code.argtypes = [i32]
            lib.orc_encode.restype = ctypes.c_uint8
            lib.orc_encode.argtypes = [i32, f32]
            lib.orc_encode_buffer.argtypes = [i32, vp, i64, vp]
            lib.orc_amax.restype = f32
            lib.orc_amax.argtypes = [vp, i32, i64]
            lib.orc_current_scale.argtypes = [f32, i32, i32, fp, fp]
            lib.orc_quantize.argtypes = [vp, i32, i64, i32, f32, vp]
            lib.orc_dequantize.argtypes = [vp, i32, i64, f32, vp]
            lib.orc_quantize_rowwise_colwise.argtypes = [vp, i32, i64, i64, i32, f32, vp, vp]
            lib.orc_quantize_block.argtypes = [vp, i32, i64, i64, i32, i64, i64, vp, vp]
            lib.orc_transpose.argtypes = [vp, i64, i64, i64, vp]
            lib.orc_delayed_update.argtypes = [vp, i32, i32, i32, f32, i64, i32, i32, i32, vp, vp]
            lib.orc_decode_buffer.argtypes = [vp, i32, i64, vp]
            lib.orc_quantize_mx.argtypes = [vp, i32, i64, i64, i32, vp, vp]
            lib.orc_num_threads.restype = i32
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle needs contiguous arrays"
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bit patterns), got %s" % x.dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


# --------------------------------------------------------------- formats ----
def decode(fmt: int, code: int) -> float:
    """Value of one code ("Megatron FP8", section 2 bit layouts and specials)."""
    return float(_load().orc_decode(fmt, int(code)))


def decode_table(fmt: int) -> np.ndarray:
    """float64[256]: the value of every code of the format."""
    return np.array([decode(fmt, c) for c in range(256)], dtype=np.float64)


def fmax(fmt: int) -> float:
    """FP8_MAX: 448 for E4M3FN, 57344 for E5M2."""
    return float(_load().orc_fmax(fmt))


def max_code(fmt: int) -> int:
    return int(_load().orc_max_code(fmt))


def encode(fmt: int, y) -> np.ndarray:
    """Saturating round-to-nearest-even encode of already-scaled float32 values."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    q = np.empty(y.shape, dtype=np.uint8)
    _load().orc_encode_buffer(fmt, _ptr(y), y.size, _ptr(q))
    return q


# ----------------------------------------------------------------- scaling ---
def amax(x: np.ndarray) -> np.float32:
    """max |x| over the tensor; NaN -> canonical NaN; empty -> 0."""
    x = np.ascontiguousarray(x)
    return np.float32(_load().orc_amax(_ptr(x), _dtype_of(x), x.size))


def current_scale(amax_value, fmt: int, margin: int = 0):
    """(scale_inv, scale) of current scaling ("Megatron FP8", sections 4 and 10)."""
    si, sc = ctypes.c_float(), ctypes.c_float()
    _load().orc_current_scale(ctypes.c_float(np.float32(amax_value)), fmt, int(margin),
                              ctypes.byref(si), ctypes.byref(sc))
    return np.float32(si.value), np.float32(sc.value)


def reciprocal(s) -> np.float32:
    """binary32 1/s, the quantizing multiplier paired with a dequant scale s."""
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        return np.float32(1.0) / np.float32(s)


def quantize(x: np.ndarray, fmt: int, scale) -> np.ndarray:
    """codes of fl32(x * scale), elementwise ("Megatron FP8", section 4)."""
    x = np.ascontiguousarray(x)
    q = np.empty(x.shape, dtype=np.uint8)
    _load().orc_quantize(_ptr(x), _dtype_of(x), x.size, fmt, ctypes.c_float(np.float32(scale)), _ptr(q))
    return q


def dequantize(q: np.ndarray, fmt: int, scale_inv) -> np.ndarray:
    """fl32(value(q) * scale_inv), elementwise."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    y = np.empty(q.shape, dtype=np.float32)
    _load().orc_dequantize(_ptr(q), fmt, q.size, ctypes.c_float(np.float32(scale_inv)), _ptr(y))
    return y


def quantize_tensor(x: np.ndarray, fmt: int, *, amax_in=None, margin: int = 0, scale_inv_in=None):
    """Per-tensor quantization with either current scaling (from ``amax_in``)
    or a given dequant scale (``scale_inv_in``, the delayed-scaling state).

    Returns dict(q, scale_inv, scale, amax) where ``amax`` is max|x| of this
    input (the value delayed scaling records after the cast)."""
    if (amax_in is None) == (scale_inv_in is None):
        raise ValueError("exactly one of amax_in / scale_inv_in")
    if amax_in is not None:
        s, sc = current_scale(amax_in, fmt, margin)
    else:
        s = np.float32(scale_inv_in)
        sc = reciprocal(s)
    return dict(q=quantize(x, fmt, sc), scale_inv=s, scale=sc, amax=amax(x))


def quantize_rowwise_colwise(x: np.ndarray, fmt: int, scale):
    """Rowwise codes [rows][cols] and columnwise codes [cols][rows] of a 2-D
    tensor with one per-tensor scale, the columnwise copy taken from the
    original input ("Hybrid quantization #2817": rowwise and columnwise
    storage, columnwise source "original")."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q_row = np.empty((rows, cols), dtype=np.uint8)
    q_col = np.empty((cols, rows), dtype=np.uint8)
    _load().orc_quantize_rowwise_colwise(_ptr(x), _dtype_of(x), rows, cols, fmt,
                                         ctypes.c_float(np.float32(scale)), _ptr(q_row), _ptr(q_col))
    return q_row, q_col


def transpose(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    xt = np.empty((cols, rows), dtype=x.dtype)
    _load().orc_transpose(_ptr(x), rows, cols, x.itemsize, _ptr(xt))
    return xt


def quantize_blocks(x: np.ndarray, fmt: int, block_rows: int, block_cols: int):
    """Codes and per-block dequant scales of block current scaling, margin 0
    ("Low Precision Training and Rollout": 128x128 block FP8 with FP32 scales)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if rows % block_rows or cols % block_cols:
        raise ValueError("blocks must tile the matrix")
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows // block_rows, cols // block_cols), dtype=np.float32)
    _load().orc_quantize_block(_ptr(x), _dtype_of(x), rows, cols, fmt, block_rows, block_cols, _ptr(q), _ptr(s))
    return q, s


def quantize_block(x: np.ndarray, fmt: int, block_rows: int):
    """Block quantization with rowwise and columnwise copies.

    block_rows 128: 128x128 blocks; block_rows 1: 1x128 blocks.  The columnwise
    copy is the same rule applied to the transposed input, so for 128x128 it
    is the transpose of the rowwise codes and scales, and for 1x128 it is a
    fresh quantization of x^T in 1x128 blocks (128 consecutive rows of one
    column of x share a scale).  Returns q_row [R][C], s_row [R/br][C/128],
    q_col [C][R], s_col [C/br][R/128]."""
    q_row, s_row = quantize_blocks(x, fmt, block_rows, 128)
    q_col, s_col = quantize_blocks(transpose(x), fmt, block_rows, 128)
    return q_row, s_row, q_col, s_col


def delayed_update(hist: np.ndarray, col: int, new_amax, step: int, fmt: int, margin: int,
                   algo: int, scale: np.ndarray, scale_inv: np.ndarray) -> None:
    """In-place delayed-scaling update of column ``col`` of ``hist``
    [history_len][n_cols] and of ``scale``/``scale_inv`` [n_cols]
    ("Megatron FP8", section 5)."""
    assert hist.dtype == np.float32 and hist.flags["C_CONTIGUOUS"] and hist.ndim == 2
    assert scale.dtype == np.float32 and scale_inv.dtype == np.float32
    L, ncols = hist.shape
    _load().orc_delayed_update(_ptr(hist), L, ncols, col, ctypes.c_float(np.float32(new_amax)), int(step),
                               fmt, int(margin), int(algo), _ptr(scale), _ptr(scale_inv))


# -------------------------------------------------------------------- GEMM ---
def quantize_mx(x: np.ndarray, fmt: int):
    """MXFP8 of a 2-D tensor along its rows ("Megatron FP8", sections 10 and 16:
    32 consecutive elements share one E8M0 power-of-two scale): returns
    (codes [rows][cols], scale bytes [rows][cols/32]).  See orc_quantize_mx for
    the shared-exponent rule."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    q = np.empty((rows, cols), dtype=np.uint8)
    sc = np.empty((rows, cols // 32), dtype=np.uint8)
    _load().orc_quantize_mx(_ptr(x), _dtype_of(x), rows, cols, fmt, _ptr(q), _ptr(sc))
    return q, sc


def quantize_mx_colwise(x: np.ndarray, fmt: int):
    """The columnwise MXFP8 copy: the same rule applied to x^T (blocks of 32
    consecutive rows of one column), as [cols][rows] codes and [cols][rows/32]
    scale bytes."""
    return quantize_mx(np.ascontiguousarray(np.asarray(x).T), fmt)


def e8m0_value(b) -> np.ndarray:
    """float64 value of E8M0 scale bytes: 2^(b - 127), NaN for 255."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def decode_codes(q: np.ndarray, fmt: int) -> np.ndarray:
    """float64 values of a code buffer."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, dtype=np.float64)
    _load().orc_decode_buffer(_ptr(q), fmt, q.size, _ptr(out))
    return out


def _mx_scaled(v: np.ndarray, scale_bytes) -> np.ndarray:
    """Element values times their block's E8M0 scale (32 per scale, along K)."""
    return v * np.repeat(e8m0_value(scale_bytes), 32, axis=1)


def _block_weight(sA, sB, mode, M, N, kb):
    """Weight of slice kb for every (m, n): sA[m,kb] * sB[., kb] with B's
    scale taken per 128-row block (128x128) or per row (1x128)."""
    sA = np.asarray(sA, dtype=np.float64)
    sB = np.asarray(sB, dtype=np.float64)
    rows_of_b = np.arange(N) // 128 if mode == BLOCK_1x128_128x128 else np.arange(N)
    return sA[:, kb][:, None] * sB[rows_of_b, kb][None, :]


def gemm_reference(A: np.ndarray, fa: int, sA, B: np.ndarray, fb: int, sB, mode: int = PER_TENSOR) -> np.ndarray:
    """float64 reference of C = (A*sA)(B*sB)^T for FP8 codes A [M][K], B [N][K].

    Per tensor: sA, sB are the two dequant scales and
    R = sA*sB * sum_k val(A[m,k]) val(B[n,k]).
    Block: sA [M][K/128] (1x128 blocks of A) and each 128-wide slice of K is
    summed on its own and weighted by the slice's two block scales,
    R = sum_kb sA[m,kb] sB[.,kb] sum_{k in kb} val(A[m,k]) val(B[n,k]),
    where sB is [N/128][K/128] (128x128 blocks of B, indexed by n // 128) or
    [N][K/128] (1x128 blocks of B, indexed by n: the weight-gradient GEMM,
    whose operands are both the transposed, token-contiguous copies).
    MXFP8: sA [M][K/32] and sB [N][K/32] are E8M0 bytes and every element is
    multiplied by its block's power of two before the products are summed.

    "Megatron FP8", section 27: products are promoted and summed at full
    precision and only the finished dot product is rounded to the output type;
    section 6: fp32 accumulation, bf16 output for fprop/dgrad and fp32 output
    for wgrad.  Here the sums are float64, in which every E4M3 x E4M3 sum at
    these sizes is exact."""
    a = decode_codes(A, fa)
    b = decode_codes(B, fb)
    if mode == PER_TENSOR:
        return (a @ b.T) * (float(np.float32(sA)) * float(np.float32(sB)))
    if mode == MXFP8:
        return _mx_scaled(a, sA) @ _mx_scaled(b, sB).T
    M, K = a.shape
    N = b.shape[0]
    R = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // 128):
        part = a[:, kb * 128:(kb + 1) * 128] @ b[:, kb * 128:(kb + 1) * 128].T
        R += part * _block_weight(sA, sB, mode, M, N, kb)
    return R


def gemm_abs_sum(A: np.ndarray, fa: int, sA, B: np.ndarray, fb: int, sB, mode: int = PER_TENSOR) -> np.ndarray:
    """S[m,n] = the same weighted sum over |val(A[m,k]) val(B[n,k])| and |weights|
    (float64): the scale of rounding error for an fp32 result.  Summing n
    terms in fp32, in any order, is off by at most (n - 1) * 2^-24 * S to first
    order (the standard bound for recursive summation)."""
    a = np.abs(decode_codes(A, fa))
    b = np.abs(decode_codes(B, fb))
    if mode == PER_TENSOR:
        return (a @ b.T) * abs(float(np.float32(sA)) * float(np.float32(sB)))
    if mode == MXFP8:
        return _mx_scaled(a, sA) @ _mx_scaled(b, sB).T
    M, K = a.shape
    N = b.shape[0]
    S = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // 128):
        part = a[:, kb * 128:(kb + 1) * 128] @ b[:, kb * 128:(kb + 1) * 128].T
        S += part * np.abs(_block_weight(sA, sB, mode, M, N, kb))
    return S


def gemm_reference_entries(A: np.ndarray, fa: int, sA, B: np.ndarray, fb: int, sB, rows, cols,
                           mode: int = PER_TENSOR) -> np.ndarray:
    """The same reference at chosen (row, col) positions only, one dot
    product per entry, for checks at sizes where the full product is too
    slow on the host."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ta = decode_table(fa)
    tb = decode_table(fb)
    out = np.empty(rows.shape[0], dtype=np.float64)
    K = A.shape[1]
    for i, (m, n) in enumerate(zip(rows, cols)):
        av = ta[A[m]]
        bv = tb[B[n]]
        if mode == PER_TENSOR:
            out[i] = float(np.dot(av, bv)) * (float(np.float32(sA)) * float(np.float32(sB)))
        elif mode == MXFP8:
            ea = np.repeat(e8m0_value(sA[m]), 32)
            eb = np.repeat(e8m0_value(sB[n]), 32)
            out[i] = float(np.dot(av * ea, bv * eb))
        else:
            acc = 0.0
            nb = n // 128 if mode == BLOCK_1x128_128x128 else n
            for kb in range(K // 128):
                sl = slice(kb * 128, (kb + 1) * 128)
                acc += float(np.dot(av[sl], bv[sl])) * float(sA[m, kb]) * float(sB[nb, kb])
            out[i] = acc
    return out


# ------------------------------------------------------------ GEMM epilogue ---
# "Megatron FP8", section 6: bias addition and an activation (ReLU, GELU) can
# be folded into the FP8 GEMM's epilogue, as Transformer Engine does for the
# MLP's bias + GELU, so the intermediate never makes a bf16 round trip;
# section 4: a tensor that is cast to FP8 records its amax for the next
# scaling decision.  The pages name the fusions but not their arithmetic; the
# readings taken here: bias is one value per output column (per output
# feature), added to the finished GEMM value; GELU is the exact form
# x * Phi(x) (Phi the standard normal CDF), not an approximation of it; ReLU
# maps values below zero to zero and keeps NaN; an FP8 output is the
# per-tensor cast (section 4) of the float32 result with a given dequant scale,
# and its amax is taken over the values before that cast.


def gelu(v) -> np.ndarray:
    """float64 GELU, x * Phi(x) = x/2 * erfc(-x / sqrt 2).  erfc (a library
    special function) keeps the relative accuracy of Phi for large negative x,
    where 1 + erf(x / sqrt 2) would cancel."""
    from scipy.special import erfc
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * erfc(-v / np.sqrt(2.0))


def relu(v) -> np.ndarray:
    """x for x >= 0 (and for NaN, and -0.0), else 0."""
    v = np.asarray(v, dtype=np.float64)
    return np.where(v < 0, 0.0, v)


def epilogue_reference(R: np.ndarray, bias=None, act: int = ACT_NONE) -> np.ndarray:
    """float64 y[m, n] = act(R[m, n] + bias[n]) for a GEMM result R [M][N]
    and a bias of one value per output column (None: no bias)."""
    y = np.asarray(R, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64).reshape(1, -1)
    if act == ACT_RELU:
        return relu(y)
    if act == ACT_GELU:
        return gelu(y)
    if act != ACT_NONE:
        raise ValueError("unknown activation %r" % act)
    return y


def epilogue_fp8_codes(y: np.ndarray, fmt: int, out_scale_inv):
    """FP8 output of the epilogue: the values rounded to float32, then the
    per-tensor cast with dequant scale s = out_scale_inv (codes of
    fl32(fl32(y) * fl32(1/s))).  Returns (codes, amax), the amax being
    max |fl32(y)| over the values before the cast."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    return quantize(y32, fmt, reciprocal(out_scale_inv)), amax(y32)



# ---------------------------------------- per-direction quantization, stats ---
COLSRC_ORIGINAL, COLSRC_ROWWISE_DEQUANTIZED = 0, 1


def _as_f32(x: np.ndarray) -> np.ndarray:
    """float32 values of a bf16 (uint16 bit patterns) or float32 tensor."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)


def quantize_hybrid(x: np.ndarray, row_fmt: int, col_fmt: int, col_source: int, *, amax_in=None,
                    row_margin: int = 0, col_margin: int = 0, row_scale_inv_in=None, col_scale_inv_in=None):
    """Per-direction ("hybrid") per-tensor quantization of a 2-D tensor
    ("[Pytorch][Common] Hybrid quantization #2817": the rowwise and the
    columnwise copies may use different formats and scaling recipes; the
    columnwise copy is quantized from the original input, or from the
    dequantized rowwise values).

    Each direction is a per-tensor quantizer of its own source: the rowwise
    source is x, the columnwise source is x (original) or
    x' = dequantize(q_row) (rowwise_dequantized).  With ``amax_in`` (current
    scaling) each direction takes the amax of its own source -- amax_in for x,
    max |x'| for x' -- with its own format and margin; otherwise the two given
    dequant scales are used.  Returns dict(q_row [R][C], q_col [C][R],
    row_scale_inv, col_scale_inv)."""
    if (amax_in is None) == (row_scale_inv_in is None or col_scale_inv_in is None):
        raise ValueError("exactly one of amax_in / the pair of given scales")
    xf = np.ascontiguousarray(_as_f32(x))
    if amax_in is not None:
        s_r, sc_r = current_scale(amax_in, row_fmt, row_margin)
    else:
        s_r = np.float32(row_scale_inv_in)
        sc_r = reciprocal(s_r)
    q_row = quantize(xf, row_fmt, sc_r)
    if col_source == COLSRC_ORIGINAL:
        src = xf
        col_amax = amax_in
    elif col_source == COLSRC_ROWWISE_DEQUANTIZED:
        src = dequantize(q_row, row_fmt, s_r)
        col_amax = None if amax_in is None else amax(src)
    else:
        raise ValueError("unknown columnwise source %r" % col_source)
    if amax_in is not None:
        s_c, sc_c = current_scale(col_amax, col_fmt, col_margin)
    else:
        s_c = np.float32(col_scale_inv_in)
        sc_c = reciprocal(s_c)
    q_col = transpose(quantize(np.ascontiguousarray(src), col_fmt, sc_c))
    return dict(q_row=q_row, q_col=q_col, row_scale_inv=s_r, col_scale_inv=s_c)


def _block_subquantizer(src: np.ndarray, recipe: int, fmt: int, pt=None):
    """(codes, scales) of one sub-quantizer applied to the rows of src; a
    per-tensor one takes its scale from pt = dict(amax_in, margin) or
    dict(scale_inv_in) and reports its dequant scale as a one-element array."""
    if recipe == SUBQ_PER_TENSOR:
        r = quantize_tensor(src, fmt, **pt)
        return r["q"], np.array([r["scale_inv"]], dtype=np.float32)
    if recipe == SUBQ_BLOCK_128x128:
        return quantize_blocks(src, fmt, 128, 128)
    if recipe == SUBQ_BLOCK_1x128:
        return quantize_blocks(src, fmt, 1, 128)
    if recipe == SUBQ_MXFP8:
        return quantize_mx(src, fmt)
    raise ValueError("unknown sub-quantizer %r" % recipe)


def _row_dequant_scales(recipe: int, s_row: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """float32 [rows][cols]: each element's dequant scale under the row recipe
    (the tensor's or its block's FP32 scale, or 2^(byte - 127) for MXFP8, NaN
    for byte 255)."""
    if recipe == SUBQ_PER_TENSOR:
        d = np.full((rows, cols), s_row[0], dtype=np.float32)
    elif recipe == SUBQ_BLOCK_128x128:
        d = np.repeat(np.repeat(s_row, 128, axis=0), 128, axis=1)
    elif recipe == SUBQ_BLOCK_1x128:
        d = np.repeat(s_row, 128, axis=1)
    else:
        d = np.repeat(e8m0_value(s_row), 32, axis=1)
    assert d.shape == (rows, cols)
    return d.astype(np.float32)


def quantize_hybrid_blockwise(x: np.ndarray, row_recipe: int, row_fmt: int, col_recipe: int, col_fmt: int,
                              col_source: int = 0, *, amax_in=None, margin: int = 0, scale_inv_in=None):
    """Per-direction ("hybrid") quantization with block sub-quantizers
    ("[Pytorch][Common] Hybrid quantization #2817": each direction has a
    quantizer of its own, format and recipe, and blockwise or MXFP8
    quantizers may fill either role; the columnwise copy is quantized from
    the original input, or from the dequantized rowwise values).

    The rowwise copy is the row recipe in row_fmt applied to x; the
    columnwise copy is the column recipe in col_fmt applied to y^T, with
    y = x (original) or y = x' = fl32(value(q_row) * d) elementwise
    (rowwise_dequantized), d the element's row-block dequant scale.  Where x'
    is NaN (a NaN row code, or a zero code times an infinite block scale) it
    is taken as the NaN carrying the row code's sign bit, so its column code
    is the NaN code with that sign (the reading of the per-tensor
    rowwise_dequantized source, extended to block scales).  A recipe is
    128x128 blocks, 1x128 blocks (both with FP32 block scales, margin 0, like
    quantize_block), MXFP8 1x32 blocks with E8M0 scales (quantize_mx), or,
    in one direction, per-tensor scaling (quantize_tensor with amax_in and
    margin, or with scale_inv_in), whose scale is reported as [s].
    Returns dict(q_row [R][C], s_row, q_col [C][R], s_col)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    pt = dict(scale_inv_in=scale_inv_in) if amax_in is None else dict(amax_in=amax_in, margin=margin)
    q_row, s_row = _block_subquantizer(x, row_recipe, row_fmt, pt)
    if col_source == COLSRC_ORIGINAL:
        src = x
    elif col_source == COLSRC_ROWWISE_DEQUANTIZED:
        v = decode_codes(q_row, row_fmt).astype(np.float32)  # exact: every code fits binary32
        with np.errstate(invalid="ignore", over="ignore", under="ignore"):
            src = v * _row_dequant_scales(row_recipe, s_row, rows, cols)
        nan = np.isnan(src)
        bits = src.view(np.uint32)
        bits[nan] = np.uint32(0x7FC00000) | ((q_row[nan].astype(np.uint32) & 0x80) << 24)
    else:
        raise ValueError("unknown columnwise source %r" % col_source)
    q_col, s_col = _block_subquantizer(transpose(np.ascontiguousarray(src)), col_recipe, col_fmt, pt)
    return dict(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col)


def cast_stats(x: np.ndarray, fmt: int, scale_inv) -> np.ndarray:
    """Diagnostics of a per-tensor cast with dequant scale s ("Megatron FP8",
    section 24: per-tensor amax, scale, overflow and underflow counts of every
    cast).  With y = fl32(x * fl32(1/s)) and c its code, returns uint64
    [overflows, underflows, nans, nonzeros]:
      overflows  -- x not NaN and |y| > FP8_MAX (the cast saturates them);
      underflows -- x finite and nonzero, and c is a zero code;
      nans       -- x is NaN;
      nonzeros   -- x not NaN and x != 0 (the population underflows are
                    counted against)."""
    xf = np.ascontiguousarray(_as_f32(x))
    with np.errstate(over="ignore", invalid="ignore"):
        y = xf * reciprocal(scale_inv)
    c = encode(fmt, y)
    nan = np.isnan(xf)
    nonzero = ~nan & (xf != 0)
    over = ~nan & (np.abs(y) > fmax(fmt))
    under = nonzero & np.isfinite(xf) & ((c & 0x7F) == 0)
    return np.array([over.sum(), under.sum(), nan.sum(), nonzero.sum()], dtype=np.uint64)


def quantize_error_feedback(g: np.ndarray, residual: np.ndarray, fmt: int, scale_inv):
    """One step of FP8 quantization with error feedback ("Megatron FP8",
    section 25: quantize g + residual, send the codes, keep what the cast lost
    for the next step):
      v = fl32(g + residual),  q = codes of fl32(v * fl32(1/s)),
      residual' = fl32(v - fl32(value(q) * s)),
    and the amax of v (what delayed scaling records for the next scale).
    Returns (q, residual', amax_v)."""
    v = (_as_f32(g) + np.asarray(residual, dtype=np.float32)).astype(np.float32)
    q = quantize(np.ascontiguousarray(v), fmt, reciprocal(scale_inv))
    with np.errstate(invalid="ignore"):
        r = (v - dequantize(q, fmt, scale_inv)).astype(np.float32)
    return q, r, amax(np.ascontiguousarray(v))
