"""GPU parity of the per-direction quantization and the diagnostics kernels
against the oracle, bit for bit:
  fp8_quantize_hybrid          ("[Pytorch][Common] Hybrid quantization #2817")
  fp8_cast_stats               ("Megatron FP8", section 24)
  fp8_quantize_error_feedback  ("Megatron FP8", section 25)
Codes, scales, residuals and counts are integers or are decided in binary32
on both sides, so every comparison is exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import empty_codes, f32_bits, first_mismatches, host, same_f32, scalar, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2
ORIG, DEQ = oracle.COLSRC_ORIGINAL, oracle.COLSRC_ROWWISE_DEQUANTIZED


def _with_specials(x: np.ndarray) -> np.ndarray:
    """Plant +-inf, NaN, zeros, a huge and a tiny value in a copy."""
    x = x.copy()
    flat = x.reshape(-1)
    if x.dtype == np.uint16:
        vals = [0x7F80, 0xFF80, 0x7FC0, 0x0000, 0x8000, 0x7F7F, 0x0001, 0xFFC0]
    else:
        vals = np.float32([np.inf, -np.inf, np.nan, 0.0, -0.0, 3e38, 1e-40, -np.nan])
    idx = np.linspace(7, flat.size - 3, len(vals)).astype(np.int64)
    flat[idx] = vals
    return x


def _input(dtype, rows, cols, seed):
    x64 = np.random.default_rng(seed).standard_normal((rows, cols)) * np.exp(
        np.random.default_rng(seed + 1).uniform(-3, 3, (1, cols)))
    if dtype == "bf16":
        return workloads.to_bf16_bits(x64)
    return x64.astype(np.float32)


def _hybrid_gpu(x, row_fmt, col_fmt, src, *, amax=None, row_margin=0, col_margin=0, s_row=None, s_col=None,
                want_row=True, want_col=True, amax_out=True):
    rows, cols = x.shape
    q_row = empty_codes((rows, cols)) if want_row else None
    q_col = empty_codes((cols, rows)) if want_col else None
    rso, cso = scalar(-1.0), scalar(-1.0)
    ao = scalar(-1.0) if amax_out else None
    fq.fp8_quantize_hybrid(to_dev(x), row_fmt, col_fmt, src, q_row=q_row, q_col=q_col,
                           amax_in=None if amax is None else scalar(float(amax)), row_margin=row_margin,
                           col_margin=col_margin, row_scale_inv_in=None if s_row is None else scalar(float(s_row)),
                           col_scale_inv_in=None if s_col is None else scalar(float(s_col)), row_scale_inv_out=rso,
                           col_scale_inv_out=cso, amax_out=ao)
    return (None if q_row is None else host(q_row), None if q_col is None else host(q_col), host(rso)[0],
            host(cso)[0], None if ao is None else host(ao)[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("src", [ORIG, DEQ])
@pytest.mark.parametrize("row_fmt,col_fmt", [(E4, E5), (E5, E4), (E4, E4), (E5, E5)])
@pytest.mark.parametrize("rows,cols", [(256, 384), (272, 400)])
def test_hybrid_current_scaling(dtype, src, row_fmt, col_fmt, rows, cols):
    x = _input(dtype, rows, cols, rows + cols + 3 * src + row_fmt)
    am = oracle.amax(x)
    want = oracle.quantize_hybrid(x, row_fmt, col_fmt, src, amax_in=am, row_margin=1, col_margin=0)
    qr, qc, rs, cs, ao = _hybrid_gpu(x, row_fmt, col_fmt, src, amax=am, row_margin=1, col_margin=0)
    assert np.array_equal(qr, want["q_row"]), first_mismatches(qr, want["q_row"])
    assert np.array_equal(qc, want["q_col"]), first_mismatches(qc, want["q_col"])
    assert f32_bits(rs) == f32_bits(want["row_scale_inv"]) and f32_bits(cs) == f32_bits(want["col_scale_inv"])
    assert f32_bits(ao) == f32_bits(am)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("src", [ORIG, DEQ])
def test_hybrid_given_scales_and_specials(dtype, src):
    """Delayed-style scales (one per direction), specials planted in the
    input: NaN codes, saturation and the dequantized source's handling of
    them must match the oracle."""
    x = _with_specials(_input(dtype, 128, 256, 9))
    s_row, s_col = np.float32(0.0123), np.float32(0.37)
    want = oracle.quantize_hybrid(x, E4, E5, src, row_scale_inv_in=s_row, col_scale_inv_in=s_col)
    qr, qc, rs, cs, ao = _hybrid_gpu(x, E4, E5, src, s_row=s_row, s_col=s_col)
    assert np.array_equal(qr, want["q_row"]), first_mismatches(qr, want["q_row"])
    assert np.array_equal(qc, want["q_col"]), first_mismatches(qc, want["q_col"])
    assert f32_bits(rs) == f32_bits(s_row) and f32_bits(cs) == f32_bits(s_col)
    assert np.isnan(ao)


def test_hybrid_single_direction_and_empty():
    x = _input("bf16", 128, 128, 21)
    am = oracle.amax(x)
    want = oracle.quantize_hybrid(x, E4, E5, DEQ, amax_in=am, row_margin=0, col_margin=1)
    _, qc, _, cs, _ = _hybrid_gpu(x, E4, E5, DEQ, amax=am, col_margin=1, want_row=False, amax_out=False)
    assert np.array_equal(qc, want["q_col"]) and f32_bits(cs) == f32_bits(want["col_scale_inv"])
    qr, _, rs, _, ao = _hybrid_gpu(x, E5, E4, ORIG, amax=am, want_col=False)
    assert np.array_equal(qr, oracle.quantize_tensor(x, E5, amax_in=am)["q"]) and f32_bits(ao) == f32_bits(am)
    # an empty tensor still publishes both scales and a zero amax
    e = np.zeros((0, 64), np.uint16)
    _, _, rs, cs, ao = _hybrid_gpu(e, E4, E5, DEQ, amax=np.float32(3.0), row_margin=2, col_margin=0)
    w = oracle.quantize_hybrid(np.zeros((16, 64), np.float32) + np.float32(3.0), E4, E5, DEQ,
                               amax_in=np.float32(3.0), row_margin=2)
    assert f32_bits(rs) == f32_bits(w["row_scale_inv"]) and f32_bits(cs) == f32_bits(w["col_scale_inv"])
    assert ao == 0.0


# ---------------------------------------------------------------- stats ----
def _stats_gpu(x, fmt, s):
    st = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    fq.fp8_cast_stats(to_dev(x), fmt, scalar(float(s)), st)
    return host(st).astype(np.uint64)


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("s", [1.0, 1e-3, 37.5, 2.0 ** -20, 3e-38, 1e38, np.inf, 0.0, np.nan, -2.5])
def test_cast_stats_every_bf16_pattern(fmt, s):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert np.array_equal(_stats_gpu(bits, fmt, s), oracle.cast_stats(bits, fmt, s))


@pytest.mark.parametrize("n", [0, 5, 1000, 4096 * 3 + 7])
def test_cast_stats_fp32_tails(n):
    x = np.float32(np.random.default_rng(n).standard_normal(n) * 300)
    if n > 8:
        x = _with_specials(x)
    for fmt in (E4, E5):
        assert np.array_equal(_stats_gpu(x, fmt, 0.5), oracle.cast_stats(x, fmt, 0.5))


def test_cast_stats_full_size_delayed_step():
    """An 8192x8192 bf16 step of the delayed-scaling workload: E4M3 under a
    scale too small for its outliers (overflows) and too coarse for its
    smallest values (underflows); E5M2's wider range, once with overflows
    only and once with underflows only."""
    x = workloads.delayed_step(7)
    for fmt, s, over, under in ((E4, 0.0005, True, True), (E5, 2e-5, True, False), (E5, 0.02, False, True)):
        got = _stats_gpu(x, fmt, s)
        want = oracle.cast_stats(x, fmt, s)
        assert np.array_equal(got, want), (got, want)
        assert (want[0] > 0) == over and (want[1] > 0) == under and want[3] == x.size


# ------------------------------------------------------- error feedback ----
def _ef_gpu(g, r, fmt, s, q_fill=0xA5):
    rd = to_dev(np.float32(r))
    q = empty_codes(g.size, q_fill)
    am = scalar(-1.0)
    fq.fp8_quantize_error_feedback(to_dev(g.reshape(-1)), rd, fmt, scalar(float(s)), q, am)
    return host(q), host(rd), host(am)[0]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("n", [16, 4096 * 5 + 9, 1 << 20])
def test_error_feedback_step(dtype, fmt, n):
    rng = np.random.default_rng(n + fmt)
    g64 = rng.standard_normal(n) * 1e-2
    g = workloads.to_bf16_bits(g64) if dtype == "bf16" else g64.astype(np.float32)
    r = np.float32(rng.standard_normal(n) * 1e-4)
    s = np.float32(2.0 ** -10 if fmt == E5 else 1e-4)
    q, rn, am = _ef_gpu(g, r, fmt, s)
    wq, wr, wam = oracle.quantize_error_feedback(g, r, fmt, s)
    assert np.array_equal(q, wq), first_mismatches(q, wq)
    assert same_f32(rn, wr)
    assert f32_bits(am) == f32_bits(wam)


def test_error_feedback_chain_and_specials():
    """Twelve steps carrying the residual on the device against the oracle's
    chain, with saturation (the clipped part is carried) and specials."""
    rng = np.random.default_rng(5)
    n = 8192 + 48
    s = np.float32(2.0 ** -12)
    r_host = np.zeros(n, np.float32)
    rd = torch.zeros(n, dtype=torch.float32, device="cuda")
    for t in range(12):
        g = workloads.to_bf16_bits(rng.standard_normal(n) * 1e-3 * (1 + 20 * (t == 4)))
        if t == 7:
            g = _with_specials(g)
        q = empty_codes(n)
        am = scalar(-1.0)
        fq.fp8_quantize_error_feedback(to_dev(g), rd, E5, scalar(float(s)), q, am)
        wq, r_host, wam = oracle.quantize_error_feedback(g, r_host, E5, s)
        assert np.array_equal(host(q), wq), (t, first_mismatches(host(q), wq))
        assert same_f32(host(rd), r_host), t
        assert same_f32(host(am), np.float32([wam])), t
