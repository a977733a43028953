"""GPU parity over a seeded sweep of shapes: ragged tile edges (multiples of 16
that are not multiples of 128), grids smaller and larger than one wave of
tiles, N a multiple of 128 but not of 256 (half-empty last tile column), for
the tile kernels (rowwise+columnwise, block, MXFP8, per-direction) and every
GEMM mode.  Codes and scales are compared bit for bit with the oracle; GEMM
outputs within the bf16 bar (1e-2 max |R|) with amax == max |C|."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import empty_codes, f32_bits, first_mismatches, host, same_f32, scalar, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2


def _x(rng, rows, cols, dt):
    v = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-4, 4, (rows, 1)))
    return v.astype(np.float32) if dt == "f32" else workloads.to_bf16_bits(v)


@pytest.mark.parametrize("seed", range(12))
def test_rowwise_colwise_and_hybrid_shapes(seed):
    rng = np.random.default_rng(1000 + seed)
    rows, cols = 16 * int(rng.integers(1, 41)), 16 * int(rng.integers(1, 41))
    dt = "bf16" if seed % 2 else "f32"
    fmt, cfmt = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    x = _x(rng, rows, cols, dt)
    a = oracle.amax(x)
    qr, qc = empty_codes((rows, cols)), empty_codes((cols, rows))
    fq.fp8_quantize_rowwise_colwise(to_dev(x), fmt, q_row=qr, q_col=qc, amax_in=scalar(a), margin=seed % 3)
    _, sc = oracle.current_scale(a, fmt, seed % 3)
    wr, wc = oracle.quantize_rowwise_colwise(x, fmt, sc)
    assert np.array_equal(host(qr), wr), (rows, cols, first_mismatches(host(qr), wr))
    assert np.array_equal(host(qc), wc), (rows, cols, first_mismatches(host(qc), wc))
    src = seed % 2
    qr, qc = empty_codes((rows, cols)), empty_codes((cols, rows))
    fq.fp8_quantize_hybrid(to_dev(x), fmt, cfmt, src, q_row=qr, q_col=qc, amax_in=scalar(a), row_margin=1)
    w = oracle.quantize_hybrid(x, fmt, cfmt, src, amax_in=a, row_margin=1)
    assert np.array_equal(host(qr), w["q_row"]) and np.array_equal(host(qc), w["q_col"]), (rows, cols)


@pytest.mark.parametrize("seed", range(10))
def test_block_and_mx_shapes(seed):
    rng = np.random.default_rng(2000 + seed)
    rows, cols = 128 * int(rng.integers(1, 7)), 128 * int(rng.integers(1, 7))
    dt = "bf16" if seed % 2 else "f32"
    fmt = int(rng.integers(0, 2))
    x = _x(rng, rows, cols, dt)
    for br in (128, 1):
        nr = rows // br
        qr, qc = empty_codes((rows, cols)), empty_codes((cols, rows))
        sr = torch.empty((nr, cols // 128), device="cuda")
        scol = torch.empty((cols // br if br == 1 else cols // 128, rows // 128), device="cuda")
        fq.fp8_quantize_block(to_dev(x), fmt, br, qr, sr, qc, scol)
        w = oracle.quantize_block(x, fmt, br)
        assert np.array_equal(host(qr), w[0]) and same_f32(host(sr), w[1]), (br, rows, cols)
        assert np.array_equal(host(qc), w[2]) and same_f32(host(scol), w[3]), (br, rows, cols)
    q, s = empty_codes((rows, cols)), empty_codes((rows, cols // 32))
    qc, sc = empty_codes((cols, rows)), empty_codes((cols, rows // 32))
    fq.fp8_quantize_mx(to_dev(x), fmt, q, s, qc, sc)
    wq, ws = oracle.quantize_mx(x, fmt)
    wqc, wsc = oracle.quantize_mx_colwise(x, fmt)
    assert np.array_equal(host(q), wq) and np.array_equal(host(s), ws), (rows, cols)
    assert np.array_equal(host(qc), wqc) and np.array_equal(host(sc), wsc), (rows, cols)


def _gemm(A, fa, sA, B, fb, sB, mode, dtype):
    M, N = A.shape[0], B.shape[0]
    C = torch.full((M, N), 7.0, dtype=dtype, device="cuda")
    am = scalar(-1.0)

    def scales(s):
        s = np.asarray(s)
        return to_dev(np.ascontiguousarray((s if s.dtype == np.uint8 else np.float32(s)).reshape(-1)))
    fq.fp8_scaled_gemm(to_dev(A), fa, scales(sA), to_dev(B), fb, scales(sB), mode, C, am)
    return host(C.float()), host(am)[0]


@pytest.mark.parametrize("seed", range(16))
def test_gemm_shapes_every_mode(seed):
    rng = np.random.default_rng(3000 + seed)
    M, N = (128 * int(rng.integers(1, 13)) for _ in range(2))
    K = 128 * int(rng.integers(1, 7))
    mode = seed % 4
    fa, fb = (E5, E4) if seed % 3 == 0 else (E4, E4)
    xa = _x(rng, M, K, "bf16")
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * 0.05)
    if mode == fq.PER_TENSOR:
        ra = oracle.quantize_tensor(xa, fa, amax_in=oracle.amax(xa))
        rb = oracle.quantize_tensor(xb, fb, amax_in=oracle.amax(xb))
        A, sA, B, sB = ra["q"], ra["scale_inv"], rb["q"], rb["scale_inv"]
    elif mode == fq.MXFP8:
        A, sA = oracle.quantize_mx(xa, fa)
        B, sB = oracle.quantize_mx(xb, fb)
    else:
        A, sA, _, _ = oracle.quantize_block(xa, fa, 1)
        B, sB, _, _ = oracle.quantize_block(xb, fb, 128 if mode == fq.BLOCK_1x128_128x128 else 1)
    dtype = torch.float32 if seed % 2 else torch.bfloat16
    C, am = _gemm(A, fa, sA, B, fb, sB, mode, dtype)
    R = oracle.gemm_reference(A, fa, sA, B, fb, sB, mode)
    err = np.max(np.abs(C.astype(np.float64) - R))
    assert err <= 1e-2 * np.max(np.abs(R)), (M, N, K, mode, err)
    assert f32_bits(am) == f32_bits(np.max(np.abs(C))), (M, N, K, mode)
