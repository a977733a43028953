"""The C-ABI library loads on a machine without a GPU, exports every entry
point the header declares, and rejects bad arguments on the host before any
HIP call (every case below fails validation, so nothing reaches the device)."""
import ctypes
import os
import re

import pytest

import oracle
from conftest import ROOT

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")

HEADER = os.path.join(ROOT, "include", "fp8q.h")
L = fq.lib
S = 0  # default stream handle (never used: every call fails validation)
BAD = 0x1000  # a 16-byte aligned fake device address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"^(?:int|const char \*)\s*(\w+)\(", text, flags=re.M))


def test_header_and_library_agree():
    names = declared_functions()
    assert names == set(fq.SIGNATURES), names ^ set(fq.SIGNATURES)
    for name in names:
        assert hasattr(L, name), name
    # the binding sets an argument list of the declared arity
    text = open(HEADER).read()
    for name in names:
        decl = re.search(r"^(?:int|const char \*)\s*%s\((.*?)\);" % name, text, flags=re.S | re.M).group(1)
        arity = 0 if decl.strip() == "void" else decl.count(",") + 1
        assert arity == len(fq.SIGNATURES[name]), name


def test_enum_values_match_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define (FP8Q_\w+) (\d+)", text))
    assert int(defs["FP8Q_E4M3FN"]) == fq.E4M3FN and int(defs["FP8Q_E5M2"]) == fq.E5M2
    assert int(defs["FP8Q_F32"]) == fq.F32 and int(defs["FP8Q_BF16"]) == fq.BF16
    assert int(defs["FP8Q_EINVAL"]) == fq.EINVAL and int(defs["FP8Q_EUNSUPPORTED"]) == fq.EUNSUPPORTED
    assert int(defs["FP8Q_PER_TENSOR"]) == fq.PER_TENSOR
    assert int(defs["FP8Q_BLOCK_1x128_128x128"]) == fq.BLOCK_1x128_128x128 == oracle.BLOCK_1x128_128x128
    assert int(defs["FP8Q_BLOCK_1x128_1x128"]) == fq.BLOCK_1x128_1x128 == oracle.BLOCK_1x128_1x128
    assert int(defs["FP8Q_MXFP8"]) == fq.MXFP8 == oracle.MXFP8
    assert int(defs["FP8Q_OUT_E4M3FN"]) == fq.OUT_E4M3FN and int(defs["FP8Q_OUT_E5M2"]) == fq.OUT_E5M2
    assert int(defs["FP8Q_ACT_NONE"]) == fq.ACT_NONE == oracle.ACT_NONE
    assert int(defs["FP8Q_ACT_RELU"]) == fq.ACT_RELU == oracle.ACT_RELU
    assert int(defs["FP8Q_ACT_GELU"]) == fq.ACT_GELU == oracle.ACT_GELU
    assert int(defs["FP8Q_COLSRC_ORIGINAL"]) == fq.COLSRC_ORIGINAL == oracle.COLSRC_ORIGINAL
    assert int(defs["FP8Q_COLSRC_ROWWISE_DEQUANTIZED"]) == fq.COLSRC_ROWWISE_DEQUANTIZED \
        == oracle.COLSRC_ROWWISE_DEQUANTIZED
    assert int(defs["FP8Q_SUBQ_BLOCK_128x128"]) == fq.SUBQ_BLOCK_128x128 == oracle.SUBQ_BLOCK_128x128
    assert int(defs["FP8Q_SUBQ_BLOCK_1x128"]) == fq.SUBQ_BLOCK_1x128 == oracle.SUBQ_BLOCK_1x128
    assert int(defs["FP8Q_SUBQ_MXFP8"]) == fq.SUBQ_MXFP8 == oracle.SUBQ_MXFP8
    assert int(defs["FP8Q_SUBQ_PER_TENSOR"]) == fq.SUBQ_PER_TENSOR == oracle.SUBQ_PER_TENSOR


def _expect(status, code, fragment):
    assert status == code, (status, fq.last_error())
    assert fragment in fq.last_error(), fq.last_error()


def test_amax_validation():
    _expect(L.fp8_amax(BAD, 7, 16, BAD, S), fq.EINVAL, "dtype")
    _expect(L.fp8_amax(BAD, fq.F32, -1, BAD, S), fq.EINVAL, "negative")
    _expect(L.fp8_amax(BAD + 4, fq.F32, 16, BAD + 0x100, S), fq.EINVAL, "16-byte")
    _expect(L.fp8_amax(None, fq.F32, 16, BAD, S), fq.EINVAL, "16-byte")
    _expect(L.fp8_amax(BAD, fq.F32, 16, None, S), fq.EINVAL, "amax")
    _expect(L.fp8_amax(BAD, fq.F32, 16, BAD + 8, S), fq.EINVAL, "overlaps")


def test_quantize_tensor_validation():
    q = BAD + 0x10000
    _expect(L.fp8_quantize_tensor(BAD, fq.BF16, 64, 5, BAD + 0x800, 0, None, q, None, None, None, S),
            fq.EINVAL, "format")
    _expect(L.fp8_quantize_tensor(BAD, fq.BF16, 64, 0, None, 0, None, q, None, None, None, S),
            fq.EINVAL, "exactly one")
    _expect(L.fp8_quantize_tensor(BAD, fq.BF16, 64, 0, BAD + 0x800, 0, BAD + 0x900, q, None, None, None, S),
            fq.EINVAL, "exactly one")
    _expect(L.fp8_quantize_tensor(BAD, fq.BF16, 64, 0, BAD + 0x800, 0, None, q, None, None, BAD + 0x800, S),
            fq.EINVAL, "aliases")
    _expect(L.fp8_quantize_tensor(BAD, fq.BF16, 64, 0, BAD + 0x800, 0, None, q + 1, None, None, None, S),
            fq.EINVAL, "q must")
    _expect(L.fp8_quantize_tensor(BAD, fq.BF16, 64, 0, BAD + 0x800, 0, None, BAD + 32, None, None, None, S),
            fq.EINVAL, "overlaps")
    _expect(L.fp8_quantize_tensor(BAD, fq.BF16, 64, 0, BAD + 0x802, 0, None, q, None, None, None, S),
            fq.EINVAL, "aligned")


def test_quantize_tensor_stats_validation():
    q, st, am = BAD + 0x10000, BAD + 0x20000, BAD + 0x800
    f = L.fp8_quantize_tensor_stats
    _expect(f(BAD, fq.BF16, 64, 0, am, 0, None, q, None, None, None, None, S), fq.EINVAL, "stats must be given")
    _expect(f(BAD, fq.BF16, 64, 0, am, 0, None, q, None, None, None, st + 4, S), fq.EINVAL, "8-byte")
    _expect(f(BAD, fq.BF16, 64, 0, am, 0, None, q, None, None, None, am - 8, S), fq.EINVAL, "stats overlaps a scalar")
    _expect(f(BAD, fq.BF16, 64, 0, am, 0, None, q, None, None, None, BAD + 64, S), fq.EINVAL, "stats overlaps x")
    _expect(f(BAD, fq.BF16, 64, 0, am, 0, None, q, None, None, None, q + 32, S), fq.EINVAL, "stats overlaps x or q")
    # the checks of fp8_quantize_tensor come first, under this call's name
    _expect(f(BAD, fq.BF16, 64, 5, am, 0, None, q, None, None, None, st, S), fq.EINVAL, "fp8_quantize_tensor_stats")
    _expect(f(BAD, fq.BF16, 64, 0, None, 0, None, q, None, None, None, st, S), fq.EINVAL, "exactly one")


def test_dequant_and_rowwise_colwise_validation():
    _expect(L.fp8_dequantize(BAD, 3, 16, BAD + 0x800, BAD + 0x1000, S), fq.EINVAL, "format")
    _expect(L.fp8_dequantize(BAD, 0, 16, None, BAD + 0x1000, S), fq.EINVAL, "scale_inv")
    _expect(L.fp8_dequantize(BAD, 0, 16, BAD + 0x800, BAD + 8, S), fq.EINVAL, "16-byte")
    rc = L.fp8_quantize_rowwise_colwise
    _expect(rc(BAD, fq.BF16, 24, 32, 0, BAD + 0x800, 0, None, BAD + 0x10000, None, None, None, None, S),
            fq.EUNSUPPORTED, "multiples of 16")
    _expect(rc(BAD, fq.BF16, 32, 32, 0, BAD + 0x800, 0, None, None, None, None, None, None, S),
            fq.EINVAL, "at least one")
    _expect(rc(BAD, fq.BF16, 32, 32, 0, BAD + 0x800, 0, None, BAD + 0x10000, BAD + 0x10010, None, None, None, S),
            fq.EINVAL, "overlap")


def test_block_and_delayed_validation():
    blk = L.fp8_quantize_block
    _expect(blk(BAD, fq.BF16, 128, 128, 0, 64, BAD + 0x10000, BAD + 0x20000, None, None, S), fq.EINVAL, "block_rows")
    _expect(blk(BAD, fq.BF16, 128, 200, 0, 128, BAD + 0x10000, BAD + 0x20000, None, None, S),
            fq.EUNSUPPORTED, "multiples of 128")
    _expect(blk(BAD, fq.BF16, 128, 128, 0, 1, BAD + 0x10000, BAD + 0x20000, BAD + 0x30000, None, S),
            fq.EINVAL, "both")
    up = L.fp8_update_scale_delayed
    _expect(up(BAD, 16, 1, 1, BAD + 0x100, 0, 0, 0, 0, BAD + 0x200, BAD + 0x300, S), fq.EINVAL, "col")
    _expect(up(BAD, 16, 1, 0, BAD + 0x100, 0, 0, 0, 9, BAD + 0x200, BAD + 0x300, S), fq.EINVAL, "algo")
    _expect(up(BAD, 16, 1, 0, BAD + 0x100, -2, 0, 0, 0, BAD + 0x200, BAD + 0x300, S), fq.EINVAL, "step")
    _expect(up(BAD, 16, 1, 0, BAD + 0x100, 0, 0, 0, 0, BAD + 0x8, BAD + 0x300, S), fq.EINVAL, "overlap")


def test_delayed_step_validation():
    d = L.fp8_quantize_delayed
    H, SC, SI, Q = BAD + 0x40, BAD + 0x200, BAD + 0x300, BAD + 0x10000
    # the history ring inside x (128 bytes of bf16), then inside q
    _expect(d(BAD, fq.BF16, 64, 0, H, 16, 1, 0, 0, 0, 0, 0, SC, SI, Q, None, None, S), fq.EINVAL, "overlap")
    _expect(d(BAD, fq.BF16, 64, 0, Q + 16, 4, 1, 0, 0, 0, 0, 0, SC, SI, Q, None, None, S), fq.EINVAL, "overlap")
    _expect(d(BAD, fq.BF16, 64, 0, BAD + 0x400, 16, 1, 0, 0, 0, 0, 0, BAD + 0x400, SI, Q, None, None, S),
            fq.EINVAL, "overlap")
    H = BAD + 0x40000
    _expect(d(BAD, fq.BF16, 64, 3, H, 16, 1, 0, 0, 0, 0, 0, SC, SI, Q, None, None, S), fq.EINVAL, "format")
    _expect(d(BAD, fq.BF16, 64, 0, H, 16, 1, 2, 0, 0, 0, 0, SC, SI, Q, None, None, S), fq.EINVAL, "col")
    _expect(d(BAD, fq.BF16, 64, 0, H, 16, 1, 0, -1, 0, 0, 0, SC, SI, Q, None, None, S), fq.EINVAL, "step")
    _expect(d(BAD, fq.BF16, 64, 0, H, 16, 1, 0, 0, 0, 0, 0, SC, SI, Q + 3, None, None, S), fq.EINVAL, "q must")
    _expect(d(BAD, fq.BF16, 64, 0, H, 16, 1, 0, 0, 0, 0, 0, SC, SI, Q, SI, None, S), fq.EINVAL, "overlap")


def test_mx_validation():
    m = L.fp8_quantize_mx
    Q, SR = BAD + 0x100000, BAD + 0x200000
    _expect(m(BAD, fq.BF16, 128, 128, 2, Q, SR, None, None, S), fq.EINVAL, "format")
    _expect(m(BAD, fq.BF16, 128, 96, 0, Q, SR, None, None, S), fq.EUNSUPPORTED, "multiples")
    _expect(m(BAD, fq.BF16, 128, 128, 0, Q, SR, Q + 0x10000, None, S), fq.EINVAL, "both")
    _expect(m(BAD, fq.BF16, 128, 128, 0, Q + 1, SR, None, None, S), fq.EINVAL, "16-byte")
    _expect(m(BAD, fq.BF16, 128, 128, 0, Q, Q + 0x100, None, None, S), fq.EINVAL, "overlap")


def test_gemm_validation():
    g = L.fp8_scaled_gemm
    A, B, C = BAD + 0x100000, BAD + 0x200000, BAD + 0x300000
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 128, 128, 128, 0, C, 7, None, S), fq.EINVAL, "dtype")
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 128, 128, 128, 4, C, fq.F32, None, S), fq.EINVAL, "mode")
    # an fp32 C of 128x128 spans 64 KiB: one that starts 32 KiB before B overlaps it
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 128, 128, 128, 2, B - 0x8000, fq.F32, None, S), fq.EINVAL, "overlaps")
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 128, 100, 128, 0, C, fq.BF16, None, S), fq.EUNSUPPORTED, "multiples")
    _expect(g(A, 2, BAD, B, 0, BAD + 4, 128, 128, 128, 0, C, fq.BF16, None, S), fq.EINVAL, "format")
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 128, 128, 128, 5, C, fq.BF16, None, S), fq.EINVAL, "mode")
    _expect(g(A, 0, None, B, 0, BAD + 4, 128, 128, 128, 0, C, fq.BF16, None, S), fq.EINVAL, "sA")
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 128, 128, 128, 0, A + 64, fq.BF16, None, S), fq.EINVAL, "overlaps")
    _expect(g(A + 8, 0, BAD, B, 0, BAD + 4, 128, 128, 128, 0, C, fq.BF16, None, S), fq.EINVAL, "16-byte")
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 128, 128, (1 << 22) + 128, 0, C, fq.BF16, None, S), fq.EUNSUPPORTED, "2^22")
    _expect(g(A, 0, BAD, B, 0, BAD + 4, 1 << 31, 1 << 31, 128, 0, C, fq.BF16, None, S), fq.EUNSUPPORTED, "tiles")


def test_gemm_fused_validation():
    g = L.fp8_scaled_gemm_fused
    A, B, C, SI, BIAS = BAD + 0x100000, BAD + 0x200000, BAD + 0x300000, BAD + 0x8, BAD + 0x400000
    E4OUT = fq.OUT_E4M3FN

    def call(bias=None, act=0, c=C, c_type=fq.BF16, si=None, amax=None, mode=0):
        return g(A, 0, BAD, B, 0, BAD + 4, 128, 128, 128, mode, bias, act, c, c_type, si, amax, S)

    _expect(call(act=3), fq.EINVAL, "activation")
    _expect(call(c_type=4), fq.EINVAL, "output type")
    _expect(call(c_type=E4OUT), fq.EINVAL, "c_scale_inv")
    _expect(call(c_type=E4OUT, si=SI + 2), fq.EINVAL, "c_scale_inv")
    _expect(call(si=SI), fq.EINVAL, "only for an FP8")
    _expect(call(bias=BIAS + 4), fq.EINVAL, "bias")
    _expect(call(mode=4), fq.EINVAL, "mode")
    # an FP8 C of 128x128 spans 16 KiB: a bias 8 KiB in overlaps it
    _expect(call(bias=C + 0x2000, c_type=E4OUT, si=SI), fq.EINVAL, "overlaps")
    _expect(call(c_type=E4OUT, si=C + 0x3000), fq.EINVAL, "overlaps")
    _expect(call(bias=BIAS, amax=BIAS + 0x100), fq.EINVAL, "amax_out overlaps")
    _expect(call(c_type=E4OUT, si=SI, amax=SI), fq.EINVAL, "amax_out overlaps")
    # the plain entry point does not take the fused output types
    _expect(L.fp8_scaled_gemm(A, 0, BAD, B, 0, BAD + 4, 128, 128, 128, 0, C, E4OUT, None, S), fq.EINVAL, "dtype")


def test_hybrid_validation():
    h = L.fp8_quantize_hybrid
    X, QR, QC, A, SR, SC = BAD, BAD + 0x100000, BAD + 0x200000, BAD + 0x300000, BAD + 0x300010, BAD + 0x300020

    def call(dtype=fq.BF16, rows=128, cols=128, rf=0, cf=1, src=0, amax=A, rsi=None, csi=None, qr=QR, qc=QC,
             rso=None, cso=None, ao=None):
        return h(X, dtype, rows, cols, rf, cf, src, amax, 0, 0, rsi, csi, qr, qc, rso, cso, ao, S)

    _expect(call(dtype=5), fq.EINVAL, "dtype")
    _expect(call(rf=2), fq.EINVAL, "format")
    _expect(call(cf=7), fq.EINVAL, "format")
    _expect(call(src=2), fq.EINVAL, "columnwise source")
    _expect(call(rows=24), fq.EUNSUPPORTED, "multiples of 16")
    _expect(call(qr=None, qc=None), fq.EINVAL, "at least one")
    _expect(call(amax=None), fq.EINVAL, "either amax_in")
    _expect(call(rsi=SR), fq.EINVAL, "either amax_in")
    _expect(call(amax=None, rsi=SR), fq.EINVAL, "either amax_in")
    _expect(call(amax=A + 2), fq.EINVAL, "aligned")
    _expect(call(rso=A), fq.EINVAL, "aliases")
    _expect(call(amax=None, rsi=SR, csi=SC, cso=SC), fq.EINVAL, "aliases")
    _expect(call(rso=SR + 0x100, cso=SR + 0x100), fq.EINVAL, "alias each other")
    _expect(call(qc=QR + 0x10), fq.EINVAL, "overlap")
    _expect(call(qr=X + 0x40), fq.EINVAL, "overlap")
    _expect(call(amax=QR + 0x40), fq.EINVAL, "overlaps a scale input")
    _expect(call(ao=QC + 0x40), fq.EINVAL, "overlaps x or the codes")


def test_hybrid_blockwise_validation():
    h = L.fp8_quantize_hybrid_blockwise
    X, QR, SR, QC, SC = BAD, BAD + 0x100000, BAD + 0x200000, BAD + 0x300000, BAD + 0x400000

    def call(dtype=fq.BF16, rows=256, cols=384, rr=fq.SUBQ_MXFP8, rf=0, cr=fq.SUBQ_BLOCK_1x128, cf=1, src=0, x=X,
             qr=QR, sr=SR, qc=QC, sc=SC, am=None, si=None):
        return h(x, dtype, rows, cols, rr, rf, qr, sr, cr, cf, src, qc, sc, am, 0, si, S)

    _expect(call(dtype=5), fq.EINVAL, "dtype")
    _expect(call(rf=2), fq.EINVAL, "format")
    _expect(call(cf=-1), fq.EINVAL, "format")
    _expect(call(rr=4), fq.EINVAL, "sub-quantizer")
    _expect(call(cr=-1), fq.EINVAL, "sub-quantizer")
    _expect(call(src=2), fq.EINVAL, "columnwise source")
    A = BAD + 0x500000
    _expect(call(rr=fq.SUBQ_PER_TENSOR, cr=fq.SUBQ_PER_TENSOR, am=A), fq.EINVAL, "two per-tensor")
    _expect(call(rr=fq.SUBQ_PER_TENSOR), fq.EINVAL, "exactly one of amax_in")
    _expect(call(rr=fq.SUBQ_PER_TENSOR, am=A, si=A + 4), fq.EINVAL, "exactly one of amax_in")
    _expect(call(am=A), fq.EINVAL, "per-tensor direction only")
    _expect(call(rr=fq.SUBQ_PER_TENSOR, am=A + 2), fq.EINVAL, "4-byte aligned")
    _expect(call(cr=fq.SUBQ_PER_TENSOR, src=1, am=A), fq.EUNSUPPORTED, "given scale_inv_in")
    _expect(call(rr=fq.SUBQ_PER_TENSOR, am=A, sr=QR + 0x10), fq.EINVAL, "overlap")
    _expect(call(cr=fq.SUBQ_PER_TENSOR, si=A, sc=A), fq.EINVAL, "overlap")
    _expect(call(rows=-128), fq.EINVAL, "negative")
    _expect(call(cols=200), fq.EUNSUPPORTED, "multiples of 128")
    _expect(call(sr=None), fq.EINVAL, "q_row and s_row")
    _expect(call(qc=None), fq.EINVAL, "q_col and s_col")
    _expect(call(qr=None, sr=None, qc=None, sc=None), fq.EINVAL, "at least one")
    _expect(call(x=None), fq.EINVAL, "x must be")
    _expect(call(qr=QR + 8), fq.EINVAL, "16-byte aligned")
    _expect(call(sc=SC + 2), fq.EINVAL, "4-byte aligned")
    _expect(call(qc=QR + 0x100), fq.EINVAL, "overlap")
    # the row scales of 256x384 MXFP8 are 256 * 12 bytes: a column scale
    # buffer starting inside them overlaps, one just past them does not
    _expect(call(sc=SR + 256 * 12 - 4), fq.EINVAL, "overlap")
    _expect(call(sr=X + 256 * 384 * 2 - 4), fq.EINVAL, "overlap")
    assert call(rows=0) == fq.OK and call(cols=0, qr=None, sr=None) == fq.OK


def test_stats_and_error_feedback_validation():
    st = L.fp8_cast_stats
    _expect(st(BAD, 3, 64, 0, BAD + 0x1000, BAD + 0x2000, S), fq.EINVAL, "dtype")
    _expect(st(BAD, 0, 64, 2, BAD + 0x1000, BAD + 0x2000, S), fq.EINVAL, "format")
    _expect(st(BAD, 0, -1, 0, BAD + 0x1000, BAD + 0x2000, S), fq.EINVAL, "negative")
    _expect(st(BAD, 0, 64, 0, None, BAD + 0x2000, S), fq.EINVAL, "scale_inv")
    _expect(st(BAD, 0, 64, 0, BAD + 0x1000, BAD + 0x2004, S), fq.EINVAL, "8-byte")
    _expect(st(BAD, 0, 64, 0, BAD + 0x1000, BAD + 0xFF8, S), fq.EINVAL, "overlaps scale_inv")
    _expect(st(BAD, 0, 64, 0, BAD + 0x1000, BAD + 0x80, S), fq.EINVAL, "overlaps x")
    _expect(st(BAD + 4, 0, 64, 0, BAD + 0x1000, BAD + 0x2000, S), fq.EINVAL, "16-byte")
    ef = L.fp8_quantize_error_feedback
    G, R, Q, SI, AM = BAD, BAD + 0x10000, BAD + 0x20000, BAD + 0x30000, BAD + 0x30010
    _expect(ef(G, 0, R, 64, 2, SI, Q, None, S), fq.EINVAL, "format")
    _expect(ef(G, 0, R, 64, 0, None, Q, None, S), fq.EINVAL, "scale_inv")
    _expect(ef(G, 0, R, 64, 0, SI, Q, SI, S), fq.EINVAL, "aliasing")
    _expect(ef(G, 0, R + 8, 64, 0, SI, Q, None, S), fq.EINVAL, "residual")
    _expect(ef(G, 0, G + 0x80, 64, 0, SI, Q, None, S), fq.EINVAL, "overlap")
    _expect(ef(G, 0, R, 64, 0, SI, R + 0x40, None, S), fq.EINVAL, "overlap")
    _expect(ef(G, 0, R, 64, 0, R + 0x20, Q, None, S), fq.EINVAL, "overlaps scale_inv")
    _expect(ef(G, 0, R, 64, 0, SI, Q, Q + 0x8, S), fq.EINVAL, "overlaps scale_inv or amax_out")


def test_last_error_is_thread_local_string():
    L.fp8_amax(BAD, 9, 16, BAD, S)
    msg = fq.last_error()
    assert isinstance(msg, str) and msg.startswith("fp8_amax")


def test_finish_poll_bound_knob_is_host_only():
    """The knob enqueues nothing (no device needed) and reports the bound that
    was in force; 0xFFFFFFFF restores the default of 2^21 rounds."""
    prev = ctypes.c_uint32(0)
    assert L.fp8q_set_finish_poll_rounds(ctypes.c_uint32(5), ctypes.byref(prev)) == 0
    start = prev.value
    assert L.fp8q_set_finish_poll_rounds(ctypes.c_uint32(0xFFFFFFFF), ctypes.byref(prev)) == 0
    assert prev.value == 5
    assert L.fp8q_set_finish_poll_rounds(ctypes.c_uint32(start), None) == 0
    assert fq.fp8q_set_finish_poll_rounds(fq.POLL_ROUNDS_DEFAULT) == start
    assert fq.fp8q_set_finish_poll_rounds(fq.POLL_ROUNDS_DEFAULT) == 1 << 21


# --------------------------------------------------------- lifecycle ------
# The library allocates no device memory: its reduction scratch is one device
# global of fixed size (64 slots of 14 KiB per device), whose address on the
# current device comes from hipGetSymbolAddress.  Both facts are visible in the
# built library without a GPU.
ALLOCATORS = ("hipMalloc", "hipFree", "hipHostMalloc", "hipHostFree", "hipExtMallocWithFlags", "hipMallocAsync",
              "hipFreeAsync", "hipMallocManaged", "hipMallocPitch", "hipMalloc3D", "hipMallocArray",
              "hipMemPoolCreate", "hipMemCreate", "hipMemAddressReserve")
SCRATCH_SLOTS, SLOT_BYTES = 64, 14336


def _nm(*flags):
    import subprocess
    out = subprocess.run(["nm", *flags, fq.LIB_PATH], capture_output=True, text=True, check=True).stdout
    return out.splitlines()


def test_library_never_allocates_device_memory():
    imported = {line.split()[-1].split("@")[0] for line in _nm("-D", "--undefined-only") if line.strip()}
    hip = sorted(s for s in imported if s.startswith("hip"))
    assert hip, "the library should import the HIP runtime"
    bad = [s for s in hip if s.startswith(ALLOCATORS)]
    assert not bad, bad
    assert "hipGetSymbolAddress" in imported


def test_reduction_scratch_is_a_fixed_device_global():
    rows = [line.split() for line in _nm("-S", "--defined-only")]
    sizes = [int(r[1], 16) for r in rows if len(r) == 4 and r[3] in ("scratch", "_ZL7scratch")]
    assert sizes == [SCRATCH_SLOTS * SLOT_BYTES], sizes


def test_header_states_the_scratch_lifecycle():
    text = " ".join(" ".join(re.sub(r"^\s*\*\s?", "", ln) for ln in open(HEADER).read().splitlines()).split())
    assert "never allocates device memory" in text
    assert "%d slots of %d KiB" % (SCRATCH_SLOTS, SLOT_BYTES // 1024) in text
    assert "more than %d streams" % SCRATCH_SLOTS in text


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="checks the error path of a machine without a GPU")
def test_valid_calls_without_a_device_return_ehip():
    """Valid arguments (fake, never dereferenced device addresses) where no
    device is usable: the call reports the runtime's error instead of
    crashing or silently doing nothing."""
    calls = [
        ("fp8_amax", lambda: L.fp8_amax(BAD, fq.BF16, 64, BAD + 0x1000, S)),
        ("fp8_quantize_tensor", lambda: L.fp8_quantize_tensor(BAD, fq.BF16, 64, 0, BAD + 0x800, 0, None,
                                                              BAD + 0x10000, None, None, None, S)),
        ("fp8_dequantize", lambda: L.fp8_dequantize(BAD, 0, 64, BAD + 0x800, BAD + 0x1000, S)),
        ("fp8_quantize_block", lambda: L.fp8_quantize_block(BAD, fq.BF16, 128, 128, 0, 128, BAD + 0x100000,
                                                            BAD + 0x200000, None, None, S)),
        ("fp8_quantize_hybrid_blockwise",
         lambda: L.fp8_quantize_hybrid_blockwise(BAD, fq.BF16, 128, 128, fq.SUBQ_MXFP8, 0, BAD + 0x100000,
                                                 BAD + 0x200000, fq.SUBQ_BLOCK_128x128, 1, 1, BAD + 0x300000,
                                                 BAD + 0x400000, None, 0, None, S)),
        ("fp8_update_scale_delayed", lambda: L.fp8_update_scale_delayed(BAD, 16, 1, 0, BAD + 0x100, 0, 0, 0, 0,
                                                                        BAD + 0x200, BAD + 0x300, S)),
        ("fp8_scaled_gemm", lambda: L.fp8_scaled_gemm(BAD + 0x100000, 0, BAD, BAD + 0x200000, 0, BAD + 4, 128, 128,
                                                      128, 0, BAD + 0x300000, fq.BF16, None, S)),
    ]
    for name, call in calls:
        status = call()
        msg = fq.last_error()
        assert status == fq.EHIP, (name, status, msg)
        assert msg.startswith(name + ":") and len(msg) > len(name) + 3, msg


def test_debug_log_lines():
    """FP8Q_DEBUG prints one stderr line per call with the entry point, its
    integer arguments and the status; without it nothing is printed."""
    import subprocess
    import sys
    code = ("import fp8_scaled_quantization_reduce_amd as fq\n"
            "fq.lib.fp8_amax(0x1000, 9, 16, 0x1000, None)\n"
            "fq.lib.fp8_dequantize(0x1000, 0, 64, 0x2000, 0x3000, None)\n")
    env = dict(os.environ, PYTHONPATH=ROOT)
    on = subprocess.run([sys.executable, "-c", code], env=dict(env, FP8Q_DEBUG="1"), capture_output=True, text=True)
    lines = [x for x in on.stderr.splitlines() if x.startswith("fp8q: ")]
    assert len(lines) == 2, on.stderr
    assert lines[0].startswith("fp8q: fp8_amax(dtype=9 n=16)") and "-> 1 fp8_amax: unknown dtype 9" in lines[0]
    assert lines[1].startswith("fp8q: fp8_dequantize(fmt=0 n=64)")
    off = subprocess.run([sys.executable, "-c", code], env=dict(env, FP8Q_DEBUG="0"), capture_output=True, text=True)
    assert "fp8q: " not in off.stderr
