"""GPU parity at sizes past 2^31 elements or bytes, where every index and
offset must be 64-bit: the amax and the cast over 2^31 + 2^20 + 7 bf16
elements, the rowwise + columnwise cast of a 65536 x 32784 bf16 tensor, the
per-direction block quantization (1x128 rows, MXFP8 columns) of a 65536 x
32896 one, and a GEMM whose A operand spans 2 GiB.  Inputs are a seeded pattern repeated over
the tensor with planted values past the 2^31 mark (so a 32-bit index would
miss or misplace them); results are compared with the oracle on the whole
amax and on sampled codes and outputs, the samples drawn across the whole
range including the tails."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f32_bits, host, scalar, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2
BIG = (1 << 31) + (1 << 20) + 7


def _pattern_bf16(n, seed):
    """n bf16 values: a 2^22-element seeded N(0,1) block repeated, each repeat
    scaled by 1/2, 1 or 2 in turn (exact in bf16) so that repeats differ."""
    block = workloads.to_bf16_bits(np.random.default_rng(seed).standard_normal(1 << 22))
    f = workloads.bf16_bits_to_f32(block)
    variants = [workloads.to_bf16_bits(f.astype(np.float64) * m) for m in (0.5, 1.0, 2.0)]
    reps = -(-n // block.size)
    out = np.empty(reps * block.size, dtype=np.uint16)
    for k in range(reps):
        out[k * block.size:(k + 1) * block.size] = variants[k % 3]
    return out[:n]


def _sample_idx(n, rng, k=200000):
    idx = rng.integers(0, n, k)
    return np.unique(np.concatenate([idx, np.arange(n - 64, n), np.arange((1 << 31) - 32, (1 << 31) + 32)]))


def test_amax_and_cast_past_2_31_elements():
    x = _pattern_bf16(BIG, 11)
    x[BIG - 5] = 0x4680          # 16384.0, the tensor's largest magnitude, in the tail
    x[(1 << 31) + 3] = 0xC67F    # -16320.0, past the 2^31 mark
    am_ref = oracle.amax(x)
    assert am_ref == 16384.0
    xd = to_dev(x)
    am = scalar(-1.0)
    fq.fp8_amax(xd, am)
    assert f32_bits(host(am)[0]) == f32_bits(am_ref)
    q = torch.empty(BIG, dtype=torch.uint8, device="cuda")
    si, am2 = scalar(-1.0), scalar(-1.0)
    fq.fp8_quantize_tensor(xd, E4, q, amax_in=am, margin=0, scale_inv_out=si, amax_out=am2)
    s_ref, sc_ref = oracle.current_scale(am_ref, E4, 0)
    assert f32_bits(host(si)[0]) == f32_bits(s_ref) and f32_bits(host(am2)[0]) == f32_bits(am_ref)
    idx = _sample_idx(BIG, np.random.default_rng(1))
    qs = q[torch.from_numpy(idx).to("cuda")]
    want = oracle.quantize(np.ascontiguousarray(x[idx]), E4, sc_ref)
    assert np.array_equal(host(qs), want)
    assert host(q[BIG - 5:BIG - 4])[0] == 0x7E and host(q[(1 << 31) + 3:(1 << 31) + 4])[0] == 0xFE


def test_rowwise_colwise_past_2_31_elements():
    rows, cols = 65536, 32784
    x = _pattern_bf16(rows * cols, 12).reshape(rows, cols)
    x[rows - 1, cols - 1] = 0x4600   # 8192.0 in the last element
    s = np.float32(8192.0 / 448)
    q_row = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    fq.fp8_quantize_rowwise_colwise(to_dev(x), E4, q_row=q_row, q_col=q_col, scale_inv_in=scalar(float(s)))
    rng = np.random.default_rng(2)
    r = np.concatenate([rng.integers(0, rows, 100000), [rows - 1, 0, rows - 1]])
    c = np.concatenate([rng.integers(0, cols, 100000), [cols - 1, cols - 1, 0]])
    want = oracle.quantize(np.ascontiguousarray(x[r, c]), E4, oracle.reciprocal(s))
    ri, ci = torch.from_numpy(r).to("cuda"), torch.from_numpy(c).to("cuda")
    assert np.array_equal(host(q_row[ri, ci]), want)
    assert np.array_equal(host(q_col[ci, ri]), want)
    assert host(q_row[rows - 1, cols - 1:])[0] == 0x7E


def test_hybrid_blockwise_two_recipes_past_2_31_elements():
    """1x128 E4M3 rows and MXFP8 E5M2 columns of a 65536 x 32896 bf16 tensor
    in one pass: sampled row segments and column blocks, the tails and the
    segments past the 2^31 mark included, against the oracle's quantizers of
    those segments."""
    rows, cols = 65536, 32896
    x = _pattern_bf16(rows * cols, 13).reshape(rows, cols)
    x[rows - 1, cols - 1] = 0x4600   # 8192.0 in the last element
    r_big = (1 << 31) // cols + 1    # a row that starts past element 2^31
    x[r_big, 5] = 0xC67F             # -16320.0
    q_row = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s_row = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda")
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    s_col = torch.empty((cols, rows // 32), dtype=torch.uint8, device="cuda")
    fq.fp8_quantize_hybrid_blockwise(to_dev(x), fq.SUBQ_BLOCK_1x128, E4, fq.SUBQ_MXFP8, E5, q_row=q_row, s_row=s_row,
                                     q_col=q_col, s_col=s_col)
    rng = np.random.default_rng(3)
    # row segments (row, segment of 128 columns)
    rr = np.concatenate([rng.integers(0, rows, 2000), [rows - 1, r_big, 0]])
    rs = np.concatenate([rng.integers(0, cols // 128, 2000), [cols // 128 - 1, 0, 0]])
    seg = x[rr[:, None], rs[:, None] * 128 + np.arange(128)]
    q_ref, s_ref = oracle.quantize_blocks(np.ascontiguousarray(seg), E4, 1, 128)
    cidx = torch.from_numpy(rs[:, None] * 128 + np.arange(128)).to("cuda")
    got_q = torch.gather(q_row[torch.from_numpy(rr).to("cuda")], 1, cidx)
    assert np.array_equal(host(got_q), q_ref)
    assert np.array_equal(f32_bits(host(s_row[torch.from_numpy(rr).to("cuda"), torch.from_numpy(rs).to("cuda")])),
                          f32_bits(s_ref[:, 0]))
    # column blocks (column, block of 32 rows)
    cc = np.concatenate([rng.integers(0, cols, 2000), [cols - 1, 5, 0]])
    cb = np.concatenate([rng.integers(0, rows // 32, 2000), [rows // 32 - 1, r_big // 32, 0]])
    blk = x[cb[:, None] * 32 + np.arange(32), cc[:, None]]
    qm_ref, sm_ref = oracle.quantize_mx(np.ascontiguousarray(blk), E5)
    ridx = torch.from_numpy(cb[:, None] * 32 + np.arange(32)).to("cuda")
    got_qc = torch.gather(q_col[torch.from_numpy(cc).to("cuda")], 1, ridx)
    assert np.array_equal(host(got_qc), qm_ref)
    assert np.array_equal(host(s_col[torch.from_numpy(cc).to("cuda"), torch.from_numpy(cb).to("cuda")]), sm_ref[:, 0])
    assert host(q_row[rows - 1, cols - 1:])[0] == 0x7E


def test_gemm_with_a_2_gib_operand():
    """A [262144][8192] E4M3 codes (2 GiB), B [256][8192]: per-tensor, bf16
    out with amax; sampled entries, including the last rows, against the
    float64 oracle within the GEMM tolerance, and the amax over the whole
    output equal to max |C|."""
    M, N, K = 262144, 256, 8192
    rng = np.random.default_rng(3)
    blk = oracle.encode(E4, np.float32(rng.standard_normal((4096, K)) * 40))
    A = np.tile(blk, (M // 4096, 1))
    A[M - 1] = oracle.encode(E4, np.float32(rng.standard_normal(K) * 200))
    B = oracle.encode(E4, np.float32(rng.standard_normal((N, K)) * 2))
    sA, sB = np.float32(0.01), np.float32(0.02)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    am = scalar(-1.0)
    fq.fp8_scaled_gemm(to_dev(A), E4, scalar(float(sA)), to_dev(B), E4, scalar(float(sB)), fq.PER_TENSOR, C, am)
    rows = np.concatenate([rng.integers(0, M, 2048), np.full(64, M - 1), np.arange(M - 64, M)])
    cols = np.concatenate([rng.integers(0, N, 2048), np.arange(64), rng.integers(0, N, 64)])
    R = oracle.gemm_reference_entries(A, E4, sA, B, E4, sB, rows, cols)
    got = (host(C[torch.from_numpy(rows).to("cuda"), torch.from_numpy(cols).to("cuda")]).astype(np.uint32) << 16)
    got = got.view(np.float32).astype(np.float64)
    Rlast = oracle.gemm_reference(A[M - 1:], E4, sA, B, E4, sB)
    assert np.max(np.abs(got - R)) <= 1e-2 * max(np.max(np.abs(R)), np.max(np.abs(Rlast)))
    cmax = np.max(np.abs(workloads.bf16_bits_to_f32(host(C))))
    assert f32_bits(host(am)[0]) == f32_bits(cmax)
