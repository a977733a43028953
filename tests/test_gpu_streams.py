"""Calls on several HIP streams at once.  The library keeps one reduction
scratch per (device, stream), so amax partials, cast statistics and the
delayed-scaling step of one stream must not see another stream's; every call
only enqueues on the stream it is given.  Each stream's results are checked
against the oracle bit for bit after the streams have run concurrently.
Streams are created at the default priority."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f32_bits, host, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2


def test_current_scaling_on_two_streams():
    """amax + current-scaled cast (+ fused statistics) of different tensors,
    launches interleaved between two streams, eight rounds each."""
    dev = "cuda"
    xs = [workloads.delayed_step(t, 2048, 4096) for t in (3, 4)]
    ws = [oracle.quantize_tensor(x, E4, amax_in=oracle.amax(x), margin=1) for x in xs]
    wst = [oracle.cast_stats(x, E4, w["scale_inv"]) for x, w in zip(xs, ws)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    xd = [to_dev(x.reshape(-1)) for x in xs]
    torch.cuda.synchronize()
    outs = []
    for k in range(2):
        with torch.cuda.stream(streams[k]):
            outs.append(dict(am=torch.full((1,), -1.0, device=dev), si=torch.full((1,), -1.0, device=dev),
                             q=torch.empty(xs[k].size, dtype=torch.uint8, device=dev),
                             st=torch.full((4,), -1, dtype=torch.int64, device=dev)))
    for _ in range(8):
        for k in range(2):
            o, s = outs[k], streams[k]
            fq.fp8_amax(xd[k], o["am"], stream=s)
            fq.fp8_quantize_tensor_stats(xd[k], E4, o["q"], o["st"], amax_in=o["am"], margin=1,
                                         scale_inv_out=o["si"], stream=s)
    torch.cuda.synchronize()
    for k in range(2):
        o = outs[k]
        assert f32_bits(host(o["am"])[0]) == f32_bits(oracle.amax(xs[k]))
        assert f32_bits(host(o["si"])[0]) == f32_bits(ws[k]["scale_inv"])
        assert np.array_equal(host(o["q"]), ws[k]["q"].reshape(-1))
        assert np.array_equal(host(o["st"]).astype(np.uint64), wst[k])


def test_delayed_scaling_on_two_streams():
    """Two independent delayed-scaling schedules (own ring, own scales), one per
    stream, their steps launched alternately: each ends in the state the oracle
    reaches for its own inputs."""
    dev = "cuda"
    T = 12
    sched = [[workloads.delayed_step(t, 512, 1024, seed_base=base) for t in range(T)] for base in (2000, 3000)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    st = []
    for k in range(2):
        with torch.cuda.stream(streams[k]):
            st.append(dict(hist=torch.zeros((8, 1), device=dev), sc=torch.ones(1, device=dev),
                           si=torch.ones(1, device=dev), am=torch.zeros(1, device=dev),
                           xs=[to_dev(x.reshape(-1)) for x in sched[k]],
                           qs=[torch.empty(sched[k][0].size, dtype=torch.uint8, device=dev) for _ in range(T)]))
    torch.cuda.synchronize()
    for t in range(T):
        for k in range(2):
            s, d = streams[k], st[k]
            fmt, fmt_next = (E4, E5) if t % 2 == 0 else (E5, E4)
            fq.fp8_quantize_delayed(d["xs"][t], fmt, d["hist"], 0, t, fmt_next, 0, fq.ALGO_MAX, d["sc"], d["si"],
                                    d["qs"][t], amax_out=d["am"], stream=s)
    torch.cuda.synchronize()
    for k in range(2):
        d = st[k]
        hist = np.zeros((8, 1), np.float32)
        sc, si = np.ones(1, np.float32), np.ones(1, np.float32)
        for t in range(T):
            fmt, fmt_next = (E4, E5) if t % 2 == 0 else (E5, E4)
            r = oracle.quantize_tensor(sched[k][t], fmt, scale_inv_in=si[0])
            assert np.array_equal(host(d["qs"][t]), r["q"].reshape(-1)), (k, t)
            oracle.delayed_update(hist, 0, r["amax"], t, fmt_next, 0, oracle.ALGO_MAX, sc, si)
        assert np.array_equal(f32_bits(host(d["hist"])), f32_bits(hist))
        assert f32_bits(host(d["si"])[0]) == f32_bits(si[0]) and f32_bits(host(d["sc"])[0]) == f32_bits(sc[0])


def test_gemms_with_output_amax_on_two_streams():
    """Per-tensor and block-scaled GEMMs with an output amax (block partials in
    the stream's scratch, then a finish kernel) launched alternately on two
    streams: each C is within the GEMM tolerance of the float64 reference and
    each amax is max |C| of its own output."""
    dev = "cuda"
    M, N, K = 512, 768, 1024
    cases = []
    for seeds in ((11, 12), (13, 14)):
        a, b = workloads.gemm_pair(M, N, K, seeds=seeds)
        qa = oracle.quantize_block(a, E4, 1)
        qb = oracle.quantize_block(b, E4, 128)
        cases.append(dict(A=qa[0], sA=qa[1], B=qb[0], sB=qb[1]))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for k in range(2):
        c = cases[k]
        with torch.cuda.stream(streams[k]):
            outs.append(dict(A=to_dev(c["A"]), sA=to_dev(c["sA"]), B=to_dev(c["B"]), sB=to_dev(c["sB"]),
                             one=torch.ones(1, device=dev),
                             Cb=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                             Cp=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                             ab=torch.full((1,), -1.0, device=dev), ap=torch.full((1,), -1.0, device=dev)))
    torch.cuda.synchronize()
    for _ in range(6):
        for k in range(2):
            o, s = outs[k], streams[k]
            fq.fp8_scaled_gemm(o["A"], E4, o["sA"], o["B"], E4, o["sB"], fq.BLOCK_1x128_128x128, o["Cb"], o["ab"],
                               stream=s)
            fq.fp8_scaled_gemm(o["A"], E4, o["one"], o["B"], E4, o["one"], fq.PER_TENSOR, o["Cp"], o["ap"],
                               stream=s)
    torch.cuda.synchronize()
    for k in range(2):
        c, o = cases[k], outs[k]
        for C, am, R in ((o["Cb"], o["ab"], oracle.gemm_reference(c["A"], E4, c["sA"], c["B"], E4, c["sB"],
                                                                    oracle.BLOCK_1x128_128x128)),
                         (o["Cp"], o["ap"], oracle.gemm_reference(c["A"], E4, 1.0, c["B"], E4, 1.0))):
            cf = C.float().cpu().numpy()
            assert np.max(np.abs(cf - R)) <= 1e-2 * np.max(np.abs(R))
            assert host(am)[0] == np.max(np.abs(cf))
