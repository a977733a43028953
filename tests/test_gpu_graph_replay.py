"""Reducing entry points captured into a HIP graph (torch.cuda.graph) and
replayed.

A captured launch keeps the arguments of its capture, so every replay of a
finishing-block launch waits for the same tag: the finishing block clears the
slots it collected, and each replay must see only its own partials.  Between
replays the test does eager work of its own (new input contents copied into
the captured buffer, a synchronization) and checks every replay against the
oracle for the input it ran on, alternating large and small amaxes so that a
replay that took the previous replay's partials would report the wrong one.
The library records no memset into the graph: its kernels carry the whole
call.  Expected values come from the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f32_bits, host, scalar

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2
SHAPE = (2048, 4096)  # 1024 producing blocks of the cast, 512 of the amax pass


def _inputs(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for r in range(count):
        mag = 100.0 if r % 2 == 0 else 0.25
        out.append(workloads.to_bf16_bits(rng.standard_normal(SHAPE) * mag))
    return out


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def test_amax_and_cast_with_amax_replayed():
    xs = _inputs(6, seed=5)
    x = torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(SHAPE, dtype=torch.uint8, device="cuda")
    am1, am2, si = scalar(-1.0), scalar(-1.0), scalar(0.5)
    x.copy_(_bf16(xs[0]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager warm-up on the capturing stream's kind of stream
        fq.fp8_amax(x, am1)
        fq.fp8_quantize_tensor(x, E4, q, scale_inv_in=si, amax_out=am2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fq.fp8_amax(x, am1)
        fq.fp8_quantize_tensor(x, E4, q, scale_inv_in=si, amax_out=am2)
    scale = oracle.reciprocal(np.float32(0.5))
    for r, xr in enumerate(xs):
        x.copy_(_bf16(xr))
        am1.fill_(-1.0)
        am2.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = f32_bits(oracle.amax(xr))
        assert f32_bits(host(am1)[0]) == want, r
        assert f32_bits(host(am2)[0]) == want, r
        assert np.array_equal(host(q), oracle.quantize(xr, E4, scale)), r


def test_delayed_step_replayed():
    """One captured delayed-scaling step (fixed ring slot 1 of 4) replayed on
    new inputs: each replay casts with the scale the previous replay left,
    records its own amax and derives the next scale from the ring."""
    xs = _inputs(5, seed=6)
    L = 4
    x = torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(SHAPE, dtype=torch.uint8, device="cuda")
    hist = torch.zeros((L, 1), dtype=torch.float32, device="cuda")
    scale, scale_inv, am, qsi = scalar(1.0), scalar(1.0), scalar(-1.0), scalar(-1.0)
    x.copy_(_bf16(xs[0]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fq.fp8_quantize_delayed(x, E4, hist, 0, 1, E4, 0, 0, scale, scale_inv, q, q_scale_inv_out=qsi,
                                amax_out=am)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fq.fp8_quantize_delayed(x, E4, hist, 0, 1, E4, 0, 0, scale, scale_inv, q, q_scale_inv_out=qsi,
                                amax_out=am)
    for r, xr in enumerate(xs):
        x.copy_(_bf16(xr))
        am.fill_(-1.0)
        h0 = host(hist)[:, 0].copy()
        s_in = host(scale_inv)[0]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a = oracle.amax(xr)
        assert f32_bits(host(am)[0]) == f32_bits(a), r
        assert f32_bits(host(qsi)[0]) == f32_bits(s_in), r
        assert np.array_equal(host(q), oracle.quantize(xr, E4, oracle.reciprocal(np.float32(s_in)))), r
        # the oracle's update of the ring as it stood before this replay
        h = np.ascontiguousarray(h0.reshape(L, 1))
        sc, sci = np.ones(1, np.float32), np.ones(1, np.float32)
        oracle.delayed_update(h, 0, a, 1, E4, 0, 0, sc, sci)
        assert np.array_equal(f32_bits(host(hist)), f32_bits(h)), r
        assert f32_bits(host(scale_inv)[0]) == f32_bits(sci[0]), r
        assert f32_bits(host(scale)[0]) == f32_bits(sc[0]), r


def test_gemm_amax_and_cast_stats_replayed():
    """The reductions folded by a following one-block kernel: a GEMM with output
    amax (tile maxima into partial slots, folded and cleared by the finish
    kernel) and the cast statistics (counts summed and cleared the same way),
    captured once and replayed on new operands and scales.  Each replay's C
    equals an eager call's on the same operands bit for bit, its amax is
    max |C| of what it emitted, C is within the GEMM tolerance of the float64
    oracle, and the counts equal the oracle's; the scales alternate by 2^8 so
    that a replay folding a previous replay's partials would report the wrong
    amax."""
    rng = np.random.default_rng(9)
    M, N, K = 512, 768, 512  # 2 x 3 tiles of 256 x 256
    A = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    B = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sA, sB = scalar(1.0), scalar(1.0)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    am = scalar(-1.0)
    x = torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda")
    si = scalar(0.01)
    st = torch.full((4,), -1, dtype=torch.int64, device="cuda")

    def codes(shape):
        v = workloads.to_bf16_bits(rng.standard_normal(shape))
        r = oracle.quantize_tensor(v, E4, amax_in=oracle.amax(v))
        return r["q"], r["scale_inv"]

    def load(r):
        a, sa = codes((M, K))
        b, sb = codes((N, K))
        sa = np.float32(sa * (256.0 if r % 2 == 0 else 1.0 / 256.0))
        xs = workloads.to_bf16_bits(rng.standard_normal(SHAPE) * (100.0 if r % 2 == 0 else 0.001))
        A.copy_(torch.from_numpy(a))
        B.copy_(torch.from_numpy(b))
        sA.fill_(float(sa))
        sB.fill_(float(sb))
        x.copy_(_bf16(xs))
        return a, sa, b, sb, xs

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fq.fp8_scaled_gemm(A, E4, sA, B, E4, sB, fq.PER_TENSOR, C, am)
        fq.fp8_cast_stats(x, E4, si, st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fq.fp8_scaled_gemm(A, E4, sA, B, E4, sB, fq.PER_TENSOR, C, am)
        fq.fp8_cast_stats(x, E4, si, st)
    for r in range(4):
        a, sa, b, sb, xs = load(r)
        am.fill_(-1.0)
        st.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        c_rep, am_rep, st_rep = host(C).copy(), host(am)[0], host(st).copy()
        C2 = torch.empty_like(C)
        am2 = scalar(-1.0)
        fq.fp8_scaled_gemm(A, E4, sA, B, E4, sB, fq.PER_TENSOR, C2, am2)
        torch.cuda.synchronize()
        assert np.array_equal(c_rep.view(np.uint16), host(C2).view(np.uint16)), r
        c32 = (c_rep.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        assert f32_bits(am_rep) == f32_bits(np.max(np.abs(c32))) == f32_bits(host(am2)[0]), r
        R = oracle.gemm_reference(a, E4, sa, b, E4, sb)
        assert np.max(np.abs(c32.astype(np.float64) - R)) <= 1e-2 * np.max(np.abs(R)), r
        assert np.array_equal(st_rep.astype(np.uint64), oracle.cast_stats(xs, E4, np.float32(0.01)).astype(np.uint64)), r


def test_hybrid_blockwise_replayed():
    """The per-direction quantization (per-tensor E4M3 rows with a given
    scale, MXFP8 E5M2 columns of the dequantized rows) captured once and
    replayed on new inputs: every replay matches the oracle for its own
    input, codes and scales bit for bit."""
    xs = _inputs(4, seed=9)
    x = torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda")
    rows, cols = SHAPE
    q_row = torch.empty(SHAPE, dtype=torch.uint8, device="cuda")
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    s_row = scalar(-1.0)
    s_col = torch.empty((cols, rows // 32), dtype=torch.uint8, device="cuda")
    si = scalar(0.05)

    def call():
        fq.fp8_quantize_hybrid_blockwise(x, fq.SUBQ_PER_TENSOR, E4, fq.SUBQ_MXFP8, E5,
                                         col_source=fq.COLSRC_ROWWISE_DEQUANTIZED, q_row=q_row, s_row=s_row,
                                         q_col=q_col, s_col=s_col, scale_inv_in=si)
    x.copy_(_bf16(xs[0]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for xr in xs:
        x.copy_(_bf16(xr))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.quantize_hybrid_blockwise(xr, oracle.SUBQ_PER_TENSOR, E4, oracle.SUBQ_MXFP8, E5,
                                                oracle.COLSRC_ROWWISE_DEQUANTIZED, scale_inv_in=np.float32(0.05))
        assert np.array_equal(host(q_row), want["q_row"]) and f32_bits(host(s_row)[0]) == f32_bits(want["s_row"][0])
        assert np.array_equal(host(q_col), want["q_col"]) and np.array_equal(host(s_col), want["s_col"])
