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
