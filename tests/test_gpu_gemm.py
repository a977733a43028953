"""GPU parity of the scaled FP8 GEMM against the float64 oracle.

Bar: max |C - R| <= 1e-2 * max |R| (fp32 accumulation, bf16 output), plus exact
checks where the arithmetic is exact: small-integer operands whose sums fit in
fp32 give bit-exact bf16 outputs, and the output amax equals max |C| over the
emitted values.  Operand codes and scales are made on the host by the oracle,
never by the HIP path."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f32_bits, host, scalar, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2
TOL = 1e-2


def bf16_to_f32(c: np.ndarray) -> np.ndarray:
    return (c.astype(np.uint32) << 16).view(np.float32)


def _gpu_gemm(A, fa, sA, B, fb, sB, mode):
    M, N = A.shape[0], B.shape[0]
    C = torch.full((M, N), 12345.0, dtype=torch.bfloat16, device="cuda")
    am = scalar(-1.0)
    def scales(s):  # E8M0 bytes (MXFP8) pass through; everything else is fp32
        s = np.asarray(s)
        return to_dev(np.ascontiguousarray((s if s.dtype == np.uint8 else np.float32(s)).reshape(-1)))
    fq.fp8_scaled_gemm(to_dev(A), fa, scales(sA), to_dev(B), fb, scales(sB), mode, C, am)
    return bf16_to_f32(host(C)), host(am)[0]


def _check_tol_and_amax(C, amax, R):
    err = np.max(np.abs(C.astype(np.float64) - R))
    assert err <= TOL * np.max(np.abs(R)), (err, np.max(np.abs(R)))
    assert f32_bits(amax) == f32_bits(np.max(np.abs(C)))


def _quantized(rng, shape, fmt, std=1.0):
    x = workloads.to_bf16_bits(rng.standard_normal(shape) * std)
    r = oracle.quantize_tensor(x, fmt, amax_in=oracle.amax(x))
    return r["q"], r["scale_inv"]


def _small_int_codes(rng, shape, fmt, top):
    """Codes of integers in [-top, top] (all exactly representable)."""
    vals = rng.integers(-top, top + 1, shape).astype(np.float32)
    return oracle.encode(fmt, vals), vals


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 384, 256), (128, 256, 1024)])
def test_gemm_exact_unit_entries(M, N, K):
    """Entries in {0, +-1}: integer sums, exact in fp32 and in bf16 for K <= 256."""
    rng = np.random.default_rng(M + N + K)
    A, av = _small_int_codes(rng, (M, K), E4, 1)
    B, bv = _small_int_codes(rng, (N, K), E4, 1)
    C, am = _gpu_gemm(A, E4, 1.0, B, E4, 1.0, fq.PER_TENSOR)
    ref = av.astype(np.float64) @ bv.astype(np.float64).T
    if K <= 256:
        assert np.array_equal(C, ref.astype(np.float32))
    R = oracle.gemm_reference(A, E4, 1.0, B, E4, 1.0)
    assert np.array_equal(R, ref)
    _check_tol_and_amax(C, am, R)


@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4), (E4, E5), (E5, E5)])
def test_gemm_epilogue_rounding_exact(fa, fb):
    """Integer operands up to 16 with K = 512: every partial sum is an integer
    below 2^24, so acc is exact in fp32 in any order, and the output must be
    bf16_RNE(fl32(fl32(sA*sB) * acc)) bit for bit."""
    rng = np.random.default_rng(11 + fa + 2 * fb)
    M, N, K = 256, 256, 512
    top = 16 if fa == E4 and fb == E4 else 8
    A, av = _small_int_codes(rng, (M, K), fa, top)
    B, bv = _small_int_codes(rng, (N, K), fb, top)
    sA, sB = np.float32(1.0 / 3.0), np.float32(0.7)
    C, am = _gpu_gemm(A, fa, sA, B, fb, sB, fq.PER_TENSOR)
    acc = (av.astype(np.float64) @ bv.astype(np.float64).T).astype(np.float32)
    alpha = np.float32(sA * sB)
    want = torch.from_numpy(acc * alpha).to(torch.bfloat16).float().numpy()
    assert np.array_equal(f32_bits(C), f32_bits(want))
    assert am == np.max(np.abs(want))


@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4), (E4, E5), (E5, E5)])
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (384, 640, 896), (512, 256, 2048)])
def test_gemm_per_tensor_parity(fa, fb, M, N, K):
    rng = np.random.default_rng(M * 3 + N * 5 + K * 7 + fa + 2 * fb)
    A, sA = _quantized(rng, (M, K), fa)
    B, sB = _quantized(rng, (N, K), fb, std=0.02)
    C, am = _gpu_gemm(A, fa, sA, B, fb, sB, fq.PER_TENSOR)
    _check_tol_and_amax(C, am, oracle.gemm_reference(A, fa, sA, B, fb, sB))


def _block_operands(rng, M, N, K, fa, fb, a_std=1.0, b_std=0.02):
    xa = workloads.to_bf16_bits(rng.standard_normal((M, K)) * a_std * np.exp(rng.uniform(-3, 3, (M, 1))))
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * b_std)
    qa, sa, _, _ = oracle.quantize_block(xa, fa, 1)
    qb, sb, _, _ = oracle.quantize_block(xb, fb, 128)
    return qa, sa, qb, sb


@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4)])
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (128, 384, 256), (256, 384, 512), (256, 256, 640), (384, 256, 1280)])
def test_gemm_block_parity(fa, fb, M, N, K):
    rng = np.random.default_rng(M + 2 * N + 3 * K + fa)
    qa, sa, qb, sb = _block_operands(rng, M, N, K, fa, fb)
    C, am = _gpu_gemm(qa, fa, sa, qb, fb, sb, fq.BLOCK_1x128_128x128)
    _check_tol_and_amax(C, am, oracle.gemm_reference(qa, fa, sa, qb, fb, sb, oracle.BLOCK_1x128_128x128))


def test_gemm_block_scales_are_applied_per_block():
    """With unit codes, block scales that differ per K block and per row must
    come out exactly as sum_kb sA[m,kb] sB[n/128,kb] * partial (all powers of two)."""
    rng = np.random.default_rng(5)
    M, N, K = 256, 256, 384
    A, av = _small_int_codes(rng, (M, K), E4, 1)
    B, bv = _small_int_codes(rng, (N, K), E4, 1)
    sa = np.float32(2.0 ** rng.integers(-3, 4, (M, K // 128)))
    sb = np.float32(2.0 ** rng.integers(-3, 4, (N // 128, K // 128)))
    C, am = _gpu_gemm(A, E4, sa, B, E4, sb, fq.BLOCK_1x128_128x128)
    R = oracle.gemm_reference(A, E4, sa, B, E4, sb, oracle.BLOCK_1x128_128x128)
    want = torch.from_numpy(R.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(C, want)


def test_gemm_k_zero_and_zero_operand():
    A = np.zeros((128, 0), np.uint8)
    B = np.zeros((256, 0), np.uint8)
    C, am = _gpu_gemm(A, E4, 1.0, B, E4, 1.0, fq.PER_TENSOR)
    assert not C.any() and am == 0.0
    rng = np.random.default_rng(1)
    A = np.zeros((128, 256), np.uint8)
    B, sB = _quantized(rng, (128, 256), E4)
    C, am = _gpu_gemm(A, E4, 2.0, B, E4, sB, fq.PER_TENSOR)
    assert not C.any() and am == 0.0


def test_gemm_deterministic():
    rng = np.random.default_rng(8)
    A, sA = _quantized(rng, (512, 1024), E4)
    B, sB = _quantized(rng, (384, 1024), E4)
    c1, a1 = _gpu_gemm(A, E4, sA, B, E4, sB, fq.PER_TENSOR)
    c2, a2 = _gpu_gemm(A, E4, sA, B, E4, sB, fq.PER_TENSOR)
    assert np.array_equal(f32_bits(c1), f32_bits(c2)) and a1 == a2


def test_gemm_per_tensor_full_size_8192():
    """8192^3 per-tensor E4M3 GEMM of current-scaled N(0,1) operands, every
    output element against the float64 oracle."""
    a, b = workloads.gemm_pair()
    ra = oracle.quantize_tensor(a, E4, amax_in=oracle.amax(a))
    rb = oracle.quantize_tensor(b, E4, amax_in=oracle.amax(b))
    del a, b
    C, am = _gpu_gemm(ra["q"], E4, ra["scale_inv"], rb["q"], E4, rb["scale_inv"], fq.PER_TENSOR)
    R = oracle.gemm_reference(ra["q"], E4, ra["scale_inv"], rb["q"], E4, rb["scale_inv"])
    _check_tol_and_amax(C, am, R)


@pytest.fixture(scope="module")
def mlp_operands():
    x, w, dy = workloads.mlp_block()
    qx, sx, _, _ = oracle.quantize_block(x, E4, 1)
    qw, sw, qwt, swt = oracle.quantize_block(w, E4, 128)
    qdy, sdy, _, _ = oracle.quantize_block(dy, E5, 1)
    return dict(qx=qx, sx=sx, qw=qw, sw=sw, qwt=qwt, swt=swt, qdy=qdy, sdy=sdy)


def test_gemm_block_full_size_fprop(mlp_operands):
    """Block-scaled fprop Y = X W^T (4096 x 14336 x 4096, E4M3 x E4M3, 1x128
    x 128x128 scales), every output element against the float64 oracle."""
    o = mlp_operands
    mode = fq.BLOCK_1x128_128x128
    C, am = _gpu_gemm(o["qx"], E4, o["sx"], o["qw"], E4, o["sw"], mode)
    _check_tol_and_amax(C, am, oracle.gemm_reference(o["qx"], E4, o["sx"], o["qw"], E4, o["sw"], mode))


def test_gemm_block_tp8_shard_fprop(mlp_operands):
    """The fprop on one GPU's share of an 8-way column-parallel layer (W rows
    0..1791: 4096 x 1792 x 4096, 112 tiles of 256x256, fewer than the CUs, so
    the whole output comes from the half-tile launch), every output element
    against the float64 oracle."""
    o = mlp_operands
    mode = fq.BLOCK_1x128_128x128
    qw, sw = np.ascontiguousarray(o["qw"][:1792]), np.ascontiguousarray(o["sw"][:14])
    C, am = _gpu_gemm(o["qx"], E4, o["sx"], qw, E4, sw, mode)
    _check_tol_and_amax(C, am, oracle.gemm_reference(o["qx"], E4, o["sx"], qw, E4, sw, mode))


def test_gemm_block_full_size_dgrad(mlp_operands):
    """Block-scaled dgrad dX = dY W (4096 x 4096 x 14336, E5M2 x E4M3, through
    W's columnwise copy), every output element against the float64 oracle."""
    o = mlp_operands
    mode = fq.BLOCK_1x128_128x128
    C, am = _gpu_gemm(o["qdy"], E5, o["sdy"], o["qwt"], E4, o["swt"], mode)
    _check_tol_and_amax(C, am, oracle.gemm_reference(o["qdy"], E5, o["sdy"], o["qwt"], E4, o["swt"], mode))


@pytest.mark.parametrize("mode", [fq.BLOCK_1x128_128x128, fq.BLOCK_1x128_1x128])
@pytest.mark.parametrize("M,N,K", [(4352, 4096, 256), (3072, 3072, 256), (256, 384, 256), (4352, 3968, 384)])
def test_gemm_block_last_wave_of_half_tiles(mode, M, N, K):
    """The block-scaled GEMM runs a last wave of tiles that is at most half
    full as a wave of 256x128 half tiles (a second launch): 17x16 tiles leave
    16 (both launches), 12x12 leave 144 (no split), 1x2 are all half tiles (the
    second half of the last tile lies past N), 17x16 with N = 3968 ends in a
    half-empty tile column.  Every case is checked in full against the
    oracle, with the output amax over all of C."""
    rng = np.random.default_rng(M + N + K + mode)
    xa = workloads.to_bf16_bits(rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1))))
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    qa, sa, _, _ = oracle.quantize_block(xa, E4, 1)
    qb, sb, _, _ = oracle.quantize_block(xb, E4, 128 if mode == fq.BLOCK_1x128_128x128 else 1)
    C, am = _gpu_gemm(qa, E4, sa, qb, E4, sb, mode)
    _check_tol_and_amax(C, am, oracle.gemm_reference(qa, E4, sa, qb, E4, sb, mode))


@pytest.mark.parametrize("mode", [fq.PER_TENSOR, fq.MXFP8])
@pytest.mark.parametrize("M,N,K", [(4352, 4096, 256), (256, 384, 256), (4352, 3968, 384)])
def test_gemm_per_tensor_and_mx_last_wave_of_half_tiles(mode, M, N, K):
    """The per-tensor / MXFP8 kernel's last wave of half tiles (see the
    block-scaled test above), against the full float64 oracle."""
    rng = np.random.default_rng(M + 2 * N + K + mode)
    xa = workloads.to_bf16_bits(rng.standard_normal((M, K)))
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    if mode == fq.MXFP8:
        qa, sa = oracle.quantize_mx(xa, E4)
        qb, sb = oracle.quantize_mx(xb, E4)
    else:
        ra = oracle.quantize_tensor(xa, E4, amax_in=oracle.amax(xa))
        rb = oracle.quantize_tensor(xb, E4, amax_in=oracle.amax(xb))
        qa, sa, qb, sb = ra["q"], ra["scale_inv"], rb["q"], rb["scale_inv"]
    C, am = _gpu_gemm(qa, E4, sa, qb, E4, sb, mode)
    _check_tol_and_amax(C, am, oracle.gemm_reference(qa, E4, sa, qb, E4, sb, mode))
