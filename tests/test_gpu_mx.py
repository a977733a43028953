"""GPU parity of MXFP8 quantization ("Megatron FP8", section 16: 1x32 blocks
with E8M0 scales) against the oracle: codes and scale bytes bit for bit, for
both formats, bf16 and fp32 inputs, the columnwise copy, and blocks that
exercise every branch of the exponent rule (zero, subnormal, huge, infinite
and NaN maxima, and the clamps at 2^-127 and 2^127)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import host, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2


def _gpu_mx(x, fmt, colwise=True):
    rows, cols = x.shape
    xd = to_dev(x)
    q = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, cols // 32), 0xA5, dtype=torch.uint8, device="cuda")
    qc = sc = None
    if colwise:
        qc = torch.full((cols, rows), 0xA5, dtype=torch.uint8, device="cuda")
        sc = torch.full((cols, rows // 32), 0xA5, dtype=torch.uint8, device="cuda")
    fq.fp8_quantize_mx(xd, fmt, q, s, qc, sc)
    out = (host(q), host(s))
    if colwise:
        out += (host(qc), host(sc))
    return out


def _expect(x, fmt, colwise=True):
    xf = x if x.dtype == np.float32 else workloads.bf16_bits_to_f32(x)
    got = _gpu_mx(x, fmt, colwise)
    q, s = oracle.quantize_mx(x, fmt)
    assert np.array_equal(got[1], s), np.argwhere(got[1] != s)[:5]
    assert np.array_equal(got[0], q), np.argwhere(got[0] != q)[:5]
    if colwise:
        qc, sc = oracle.quantize_mx_colwise(x, fmt)
        assert np.array_equal(got[3], sc), np.argwhere(got[3] != sc)[:5]
        assert np.array_equal(got[2], qc), np.argwhere(got[2] != qc)[:5]
    return xf


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (512, 256)])
def test_mx_bf16_matches_oracle(fmt, rows, cols):
    rng = np.random.default_rng(rows + cols + fmt)
    x = workloads.to_bf16_bits(rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-12, 12, (rows, 1))))
    _expect(x, fmt)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_mx_fp32_matches_oracle(fmt):
    rng = np.random.default_rng(7 + fmt)
    x = np.float32(rng.standard_normal((256, 256)) * np.exp(rng.uniform(-30, 30, (256, 256))))
    _expect(x, fmt)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_mx_special_blocks(fmt):
    """Zero, subnormal, near-max, infinite and NaN blocks, and the exponent
    clamps (a block max of 2^-140 clamps to e = -127; 2^127 and above clamp to
    e = 127 for E5M2's emax)."""
    rng = np.random.default_rng(17)
    x = np.float32(rng.standard_normal((128, 256)))
    x[0, :32] = 0.0                                   # all-zero row block
    x[1, :32] = np.float32(2.0 ** -140) * rng.standard_normal(32)  # subnormal maxima
    x[2, :32] = np.float32(3.0e38)                     # huge
    x[3, 5] = np.inf                                   # infinite max
    x[4, 40] = np.nan                                  # NaN block
    x[5, 64:96] = -np.float32(2.0 ** 127)
    x[:, 128] = np.float32(2.0 ** -149)                # a column of the smallest subnormal
    x[32:64, 200] = np.nan                             # a NaN column block
    _expect(x, fmt)


def test_mx_rowwise_only_and_full_size():
    """The MXFP8 operands of the 8192^3 GEMM: rowwise only at full size."""
    rng = np.random.default_rng(19)
    x = workloads.to_bf16_bits(rng.standard_normal((8192, 8192)).astype(np.float32))
    q, s = _gpu_mx(x, E4, colwise=False)
    rows = rng.integers(0, 8192, 64)
    rq, rs = oracle.quantize_mx(x[rows], E4)
    assert np.array_equal(q[rows], rq) and np.array_equal(s[rows], rs)


def test_mx_quantize_then_gemm_matches_oracle():
    """MXFP8 codes from the GPU feed the MXFP8 GEMM; the result matches the
    oracle's GEMM of the oracle's codes (which are bitwise the same)."""
    rng = np.random.default_rng(23)
    M, N, K = 256, 384, 512
    xa = workloads.to_bf16_bits(rng.standard_normal((M, K)))
    xb = workloads.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    qa, sa = _gpu_mx(xa, E4, colwise=False)
    qb, sb = _gpu_mx(xb, E4, colwise=False)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fq.fp8_scaled_gemm(to_dev(qa), E4, to_dev(sa), to_dev(qb), E4, to_dev(sb), fq.MXFP8, C)
    oa, osa = oracle.quantize_mx(xa, E4)
    ob, osb = oracle.quantize_mx(xb, E4)
    R = oracle.gemm_reference(oa, E4, osa, ob, E4, osb, oracle.MXFP8)
    S = oracle.gemm_abs_sum(oa, E4, osa, ob, E4, osb, oracle.MXFP8)
    assert np.all(np.abs(host(C) - R) <= (2.0 ** -11 + (K + 2) * 2.0 ** -24) * S)
