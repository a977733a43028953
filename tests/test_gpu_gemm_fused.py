"""GPU parity of the fused GEMM epilogue ("Megatron FP8", section 6: bias and
ReLU / GELU folded into the FP8 GEMM's epilogue; section 4: an FP8 output cast
with its own scale, whose amax feeds the next scaling decision), through
fp8_scaled_gemm_fused, against the oracle's epilogue_reference.

Error model.  The kernel's pre-activation value v + bias differs from the
float64 R + bias by at most
    e_pre = (2^-11 + (K + K/128 + 2) 2^-24) S + 2^-23 |R + bias|
(S = oracle.gemm_abs_sum: the matrix instruction's adder, fp32 summation, the
scale and the bias add).  ReLU passes errors through unchanged; GELU grows
them by at most its largest slope, 1.13 (pinned in the oracle tests), and adds
its own binary32 evaluation error, bounded here by 2^-20 |R + bias| (the
kernel's evaluation is within 2^-21.6 |x| of x Phi(x); test_gelu_dense_grid
checks that bound on its own).  Then:
  fp32 output   |C - Y| <= e
  bf16 output   |C - Y| <= e + 2^-8 (|Y| + e)        (one RNE rounding)
  FP8 output    the code lies between the codes of (Y - e) * scale and
                (Y + e) * scale (the cast is monotone), and equals the oracle's
                code wherever that interval holds a single code;
                amax_out within [max(|Y| - e), max(|Y| + e)], and the largest
                code magnitude is exactly the code of amax_out * scale.
Where every step is exact (small integers, power-of-two scales, no GELU) the
outputs, codes and amax must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f32_bits, host, scalar, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2
NONE, RELU, GELU = oracle.ACT_NONE, oracle.ACT_RELU, oracle.ACT_GELU
MFMA_ADDER = 2.0 ** -11
GELU_SLOPE = 1.13
GELU_EVAL = 2.0 ** -20
OUTS = ("f32", "bf16", "e4m3", "e5m2")
OUT_FMT = {"e4m3": E4, "e5m2": E5}


def _fused(A, fa, sA, B, fb, sB, mode, out, bias=None, act=NONE, s_out=None):
    M, N = A.shape[0], B.shape[0]
    if out in OUT_FMT:
        C = torch.full((M, N), 0xA5, dtype=torch.uint8, device="cuda")
    else:
        C = torch.full((M, N), 12345.0, dtype=torch.float32 if out == "f32" else torch.bfloat16, device="cuda")
    am = scalar(-1.0)
    sa = to_dev(np.ascontiguousarray(sA).reshape(-1))
    sb = to_dev(np.ascontiguousarray(sB).reshape(-1))
    b = None if bias is None else to_dev(np.ascontiguousarray(bias, dtype=np.float32))
    si = scalar(float(s_out)) if out in OUT_FMT else None
    fq.fp8_scaled_gemm_fused(to_dev(A), fa, sa, to_dev(B), fb, sb, mode, C, bias=b, act=act,
                             out_fmt=OUT_FMT.get(out), c_scale_inv=si, amax_out=am)
    c = host(C if out in OUT_FMT else C.float())
    return c, host(am)[0]


def _reference(A, fa, sA, B, fb, sB, mode, bias, act):
    K = A.shape[1]
    R = oracle.gemm_reference(A, fa, sA, B, fb, sB, mode)
    S = oracle.gemm_abs_sum(A, fa, sA, B, fb, sB, mode)
    pre = np.abs(R if bias is None else R + np.float64(bias)[None, :])
    e = (MFMA_ADDER + (K + K // 128 + 2) * 2.0 ** -24) * S + 2.0 ** -23 * pre
    if act == GELU:
        e = GELU_SLOPE * e + GELU_EVAL * pre
    return oracle.epilogue_reference(R, None if bias is None else np.float64(bias), act), e


def _check_float(C, am, Y, e, out):
    err = np.abs(C.astype(np.float64) - Y)
    bound = e if out == "f32" else e + 2.0 ** -8 * (np.abs(Y) + e)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (worst, err[worst], bound[worst], Y[worst])
    assert f32_bits(am) == f32_bits(np.max(np.abs(C)))


def _decode_interval(fmt, lo, hi):
    """Values of the codes of the float64 ends, each end first moved outward
    by 2^-21 of itself (covers the fp32 product's rounding)."""
    lo = (lo - 2.0 ** -21 * np.abs(lo)).astype(np.float32)
    hi = (hi + 2.0 ** -21 * np.abs(hi)).astype(np.float32)
    return oracle.decode_codes(oracle.encode(fmt, lo), fmt), oracle.decode_codes(oracle.encode(fmt, hi), fmt)


def _check_codes(q, am, Y, e, fmt, s_out):
    scale = oracle.reciprocal(s_out)
    dlo, dhi = _decode_interval(fmt, (Y - e) * float(scale), (Y + e) * float(scale))
    d = oracle.decode_codes(q, fmt)
    bad = ~((d >= dlo) & (d <= dhi))
    assert not bad.any(), (np.argwhere(bad)[:4], d[bad][:4], dlo[bad][:4], dhi[bad][:4])
    want, _ = oracle.epilogue_fp8_codes(Y, fmt, s_out)
    single = (dlo == dhi) & (dlo != 0)
    assert np.array_equal(q[single], want[single])
    # the bound above is loose (the adder term is a worst case): in practice
    # the kernel's value and the float64 one straddle a rounding boundary of
    # the FP8 grid only rarely, so nearly every code is the oracle's
    same = np.mean(q == want)
    assert same > 0.95, same
    a = np.abs(Y)
    assert np.max(a - e) <= am <= np.max(a + e), (am, np.max(a))
    top = oracle.decode_codes(oracle.encode(fmt, np.array([np.float32(am) * scale], dtype=np.float32)), fmt)[0]
    assert np.max(np.abs(d)) == top


def _check(C, am, Y, e, out, s_out):
    if out in OUT_FMT:
        _check_codes(C, am, Y, e, OUT_FMT[out], s_out)
    else:
        _check_float(C, am, Y, e, out)


def _output_scale(Y, out):
    """A dequant scale that puts max |Y| just inside the format's range."""
    if out not in OUT_FMT:
        return None
    return np.float32(np.max(np.abs(Y)) * 1.05 / oracle.fmax(OUT_FMT[out]))


# ------------------------------------------------------------ operands ----
def _pt_operands(rng, M, N, K, fa, fb):
    xa = workloads.to_bf16_bits(rng.standard_normal((M, K)))
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    ra = oracle.quantize_tensor(xa, fa, amax_in=oracle.amax(xa))
    rb = oracle.quantize_tensor(xb, fb, amax_in=oracle.amax(xb))
    return ra["q"], np.float32(ra["scale_inv"]), rb["q"], np.float32(rb["scale_inv"])


def _block_operands(rng, M, N, K, fa, fb, mode):
    xa = workloads.to_bf16_bits(rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1))))
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    qa, sa, _, _ = oracle.quantize_block(xa, fa, 1)
    qb, sb, _, _ = oracle.quantize_block(xb, fb, 128 if mode == oracle.BLOCK_1x128_128x128 else 1)
    return qa, sa, qb, sb


def _mx_operands(rng, M, N, K, fa, fb):
    xa = workloads.to_bf16_bits(rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1))))
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    qa, sa = oracle.quantize_mx(xa, fa)
    qb, sb = oracle.quantize_mx(xb, fb)
    return qa, sa, qb, sb


def _operands(rng, mode, M, N, K, fa, fb):
    if mode == oracle.PER_TENSOR:
        return _pt_operands(rng, M, N, K, fa, fb)
    if mode == oracle.MXFP8:
        return _mx_operands(rng, M, N, K, fa, fb)
    return _block_operands(rng, M, N, K, fa, fb, mode)


MODES = (oracle.PER_TENSOR, oracle.BLOCK_1x128_128x128, oracle.BLOCK_1x128_1x128, oracle.MXFP8)


# --------------------------------------------------------------- tests ----
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("act", (NONE, RELU))
def test_fused_exact_small_integers(out, mode, act):
    """Integer codes up to 8, power-of-two scales, K = 256 and biases that
    are multiples of 1/2: every sum is exact in fp32 in any order, so the
    outputs, codes and amax must match the oracle bit for bit."""
    rng = np.random.default_rng(17 + 5 * mode + 3 * act + OUTS.index(out))
    M, N, K = 256, 384, 256
    A = oracle.encode(E4, rng.integers(-8, 9, (M, K)).astype(np.float32))
    B = oracle.encode(E4, rng.integers(-8, 9, (N, K)).astype(np.float32))
    if mode == oracle.PER_TENSOR:
        sA, sB = np.float32(0.5), np.float32(0.25)
    elif mode == oracle.MXFP8:
        sA = rng.integers(126, 128, (M, K // 32)).astype(np.uint8)
        sB = rng.integers(126, 128, (N, K // 32)).astype(np.uint8)
    else:
        nb = N // 128 if mode == oracle.BLOCK_1x128_128x128 else N
        sA = np.float32(rng.choice([0.5, 0.25], (M, K // 128)))
        sB = np.float32(rng.choice([0.5, 0.25], (nb, K // 128)))
    bias = np.float32(rng.integers(-60, 61, N) + 0.5)
    Y = oracle.epilogue_reference(oracle.gemm_reference(A, E4, sA, B, E4, sB, mode), np.float64(bias), act)
    s_out = np.float32({"e4m3": 64.0, "e5m2": 2.0}.get(out, 1.0))
    C, am = _fused(A, E4, sA, B, E4, sB, mode, out, bias, act, s_out)
    if out in OUT_FMT:
        want, want_am = oracle.epilogue_fp8_codes(Y, OUT_FMT[out], s_out)
        assert np.array_equal(C, want)
        assert f32_bits(am) == f32_bits(want_am)
    else:
        want = Y.astype(np.float32)
        if out == "bf16":
            want = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
        assert np.array_equal(f32_bits(C), f32_bits(want))
        assert f32_bits(am) == f32_bits(np.max(np.abs(want)))


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("mode", MODES)
def test_fused_bias_gelu_parity(out, mode):
    rng = np.random.default_rng(101 + 7 * mode + OUTS.index(out))
    M, N, K = 384, 640, 896
    fa, fb = (E4, E4) if mode != oracle.BLOCK_1x128_1x128 else (E5, E4)
    A, sA, B, sB = _operands(rng, mode, M, N, K, fa, fb)
    R0 = oracle.gemm_reference(A[:64], fa, sA if mode == oracle.PER_TENSOR else sA[:64], B, fb, sB, mode)
    bias = np.float32(rng.standard_normal(N) * np.std(R0))
    Y, e = _reference(A, fa, sA, B, fb, sB, mode, bias, GELU)
    s_out = _output_scale(Y, out)
    C, am = _fused(A, fa, sA, B, fb, sB, mode, out, bias, GELU, s_out)
    _check(C, am, Y, e, out, s_out)


@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4), (E4, E5), (E5, E5)])
@pytest.mark.parametrize("act", (RELU, GELU))
def test_fused_formats_per_tensor(fa, fb, act):
    rng = np.random.default_rng(31 + fa + 2 * fb + 4 * act)
    M, N, K = 256, 512, 1024
    A, sA, B, sB = _pt_operands(rng, M, N, K, fa, fb)
    bias = np.float32(rng.standard_normal(N) * 0.05)
    Y, e = _reference(A, fa, sA, B, fb, sB, oracle.PER_TENSOR, bias, act)
    for out in ("bf16", "e4m3"):
        s_out = _output_scale(Y, out)
        C, am = _fused(A, fa, sA, B, fb, sB, oracle.PER_TENSOR, out, bias, act, s_out)
        _check(C, am, Y, e, out, s_out)


@pytest.mark.parametrize("out", ("bf16", "e4m3"))
def test_fused_activation_without_bias_and_bias_without_activation(out):
    rng = np.random.default_rng(5)
    M, N, K = 128, 256, 384
    A, sA, B, sB = _pt_operands(rng, M, N, K, E4, E4)
    bias = np.float32(rng.standard_normal(N) * 0.1)
    for b, act in ((None, GELU), (bias, NONE), (None, RELU)):
        Y, e = _reference(A, E4, sA, B, E4, sB, oracle.PER_TENSOR, b, act)
        s_out = _output_scale(Y, out)
        C, am = _fused(A, E4, sA, B, E4, sB, oracle.PER_TENSOR, out, b, act, s_out)
        _check(C, am, Y, e, out, s_out)


@pytest.mark.parametrize("mode", (oracle.PER_TENSOR, oracle.BLOCK_1x128_128x128))
def test_fused_k_zero_gives_activation_of_bias(mode):
    """K = 0: every row is act(bias), exactly (GELU within its evaluation
    bound), and the FP8 codes are the oracle's cast of those values."""
    M, N = 256, 384
    rng = np.random.default_rng(9)
    bias = np.float32(rng.standard_normal(N) * 3)
    A = np.zeros((M, 0), np.uint8)
    B = np.zeros((N, 0), np.uint8)
    sA = np.float32(1.0) if mode == oracle.PER_TENSOR else np.zeros((M, 0), np.float32)
    sB = np.float32(1.0) if mode == oracle.PER_TENSOR else np.zeros((N // 128, 0), np.float32)
    sa_dev = np.ones(1, np.float32) if mode != oracle.PER_TENSOR else sA
    sb_dev = np.ones(1, np.float32) if mode != oracle.PER_TENSOR else sB
    C, am = _fused(A, E4, sa_dev, B, E4, sb_dev, mode, "f32", bias, RELU)
    want = np.broadcast_to(np.where(bias < 0, np.float32(0), bias), (M, N))
    assert np.array_equal(f32_bits(C), f32_bits(want)) and am == np.max(want)
    C, am = _fused(A, E4, sa_dev, B, E4, sb_dev, mode, "e4m3", bias, NONE, np.float32(0.5))
    want, want_am = oracle.epilogue_fp8_codes(np.broadcast_to(np.float64(bias), (M, N)), E4, np.float32(0.5))
    assert np.array_equal(C, want) and f32_bits(am) == f32_bits(want_am)
    C, am = _fused(A, E4, sa_dev, B, E4, sb_dev, mode, "f32", bias, GELU)
    g = oracle.gelu(np.float64(bias))
    assert np.all(np.abs(C - g[None, :]) <= GELU_EVAL * np.abs(np.float64(bias))[None, :])


def test_gelu_dense_grid():
    """The epilogue's GELU alone (K = 0, so the pre-activation is the bias):
    61440 values over [-16, 16] and a log-spaced sweep of both signs from
    1e-30 to 1e4, against x Phi(x) in float64; then the special values."""
    grid = np.linspace(-16, 16, 65536 - 4096)
    logs = np.logspace(-30, 4, 2048)
    x = np.float32(np.concatenate([grid, logs, -logs]))
    C, _ = _fused(np.zeros((128, 0), np.uint8), E4, np.float32(1.0), np.zeros((x.size, 0), np.uint8), E4,
                  np.float32(1.0), oracle.PER_TENSOR, "f32", x, GELU)
    want = oracle.gelu(np.float64(x))
    err = np.abs(C[0].astype(np.float64) - want)
    worst = int(np.argmax(err / np.abs(np.float64(x))))
    assert np.all(err <= 2.0 ** -21 * np.abs(np.float64(x))), (x[worst], C[0][worst], want[worst])
    assert np.array_equal(f32_bits(C[0]), f32_bits(C[77]))
    # left tail: relative accuracy down to the smallest normal results
    tail = (x < -1) & (np.abs(want) > 2.0 ** -120)
    rel = np.abs(C[0][tail] - want[tail]) / np.abs(want[tail])
    assert rel.max() < 2.0 ** -14, rel.max()
    special = np.float32([np.inf, -np.inf, np.nan, 0.0, 3.4e38, -3.4e38] + [1.0] * 122)
    C, _ = _fused(np.zeros((128, 0), np.uint8), E4, np.float32(1.0), np.zeros((128, 0), np.uint8), E4,
                  np.float32(1.0), oracle.PER_TENSOR, "f32", special, GELU)
    got = C[0][:6]
    assert got[0] == np.inf and np.isnan(got[1]) and np.isnan(got[2]) and got[3] == 0
    assert got[4] == np.float32(3.4e38) and got[5] == 0


def test_fused_deterministic_and_nan_free_fp8_output():
    rng = np.random.default_rng(12)
    M, N, K = 512, 512, 512
    A, sA, B, sB = _pt_operands(rng, M, N, K, E4, E4)
    bias = np.float32(rng.standard_normal(N))
    first = _fused(A, E4, sA, B, E4, sB, oracle.PER_TENSOR, "e4m3", bias, GELU, np.float32(0.01))
    again = _fused(A, E4, sA, B, E4, sB, oracle.PER_TENSOR, "e4m3", bias, GELU, np.float32(0.01))
    assert np.array_equal(first[0], again[0]) and f32_bits(first[1]) == f32_bits(again[1])
    assert not np.any((first[0] & 0x7F) == 0x7F)


def test_fused_full_size_mlp_fc1():
    """The MLP's first projection at its full size, H = GELU(X W^T + b) with
    X 4096x4096 and W 14336x4096 (per-tensor current-scaled E4M3), emitted as
    E4M3 codes with a given output scale: sampled entries against the oracle
    and the exact amax / largest-code property over the whole output."""
    x, w, _ = workloads.mlp_block()
    ra = oracle.quantize_tensor(x, E4, amax_in=oracle.amax(x))
    rb = oracle.quantize_tensor(w, E4, amax_in=oracle.amax(w))
    del x, w
    A, sA, B, sB = ra["q"], np.float32(ra["scale_inv"]), rb["q"], np.float32(rb["scale_inv"])
    M, N, K = A.shape[0], B.shape[0], A.shape[1]
    rng = np.random.default_rng(44)
    bias = np.float32(rng.standard_normal(N) * 0.5)
    s_out = np.float32(6.0 / 448)
    C, am = _fused(A, E4, sA, B, E4, sB, oracle.PER_TENSOR, "e4m3", bias, GELU, s_out)
    rows = rng.integers(0, M, 1024)
    cols = rng.integers(0, N, 1024)
    R = oracle.gemm_reference_entries(A, E4, sA, B, E4, sB, rows, cols)
    a = np.abs(oracle.decode_table(E4))
    Sabs = np.array([float(np.dot(a[A[m]], a[B[n]])) for m, n in zip(rows, cols)]) * (float(sA) * float(sB))
    pre = np.abs(R + np.float64(bias[cols]))
    e = GELU_SLOPE * ((MFMA_ADDER + (K + K // 128 + 2) * 2.0 ** -24) * Sabs + 2.0 ** -23 * pre) + GELU_EVAL * pre
    Y = oracle.gelu(R + np.float64(bias[cols]))
    scale = oracle.reciprocal(s_out)
    dlo, dhi = _decode_interval(E4, (Y - e) * float(scale), (Y + e) * float(scale))
    d = oracle.decode_codes(C[rows, cols], E4)
    assert np.all((d >= dlo) & (d <= dhi))
    dall = oracle.decode_codes(C, E4)
    top = oracle.decode_codes(oracle.encode(E4, np.array([np.float32(am) * scale], dtype=np.float32)), E4)[0]
    assert np.max(np.abs(dall)) == top
    assert np.max(Y - e) <= am
