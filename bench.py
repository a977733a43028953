"""Benchmark of the FP8 scaled-quantization hot path on one MI355X.

Headline workload (one "step" = one pass of the path over one batch): the
delayed-scaling schedule on 8192x8192 bf16 tensors -- each step casts its
tensor to FP8 with the stored scale (E4M3FN on even steps, E5M2 on odd
steps) with the input amax fused into the same pass, then updates the
amax-history ring (length 16, max) and derives the next scale.  The 32
distinct inputs (4 GiB) are resident in HBM before timing and cycled, so the
256 MB last-level cache cannot serve repeats.

value = algorithmic bytes moved per step (2 B read + 1 B written per element)
/ time, in GB/s, the time taken from two HIP events around the timed steps on
the stream they run on.  One step is one launch of the fused entry point (the
cast kernel and the one-block ring update behind it), so the roofline object
uses that same per-step duration.

Every other row of the hot path (amax, current scaling, dequantize, rowwise +
columnwise, 128x128 and 1x128 block quantization, per-tensor and block-scaled
GEMMs, and the next rows: the fp32-output weight-gradient GEMM, MXFP8
quantization and the MXFP8 GEMM) is timed at its own workload size and
reported under "rows".

The CPU oracle is timed on the host cores on a bounded sample of the same
workload ("cpu_baseline").
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0
# HBM bytes of one delayed step (cast_kernel + delayed_kernel), from the
# FETCH_SIZE and WRITE_SIZE counters of the current kernels scaled by the
# factors a plain copy gives (profiles/delayed_step_8192x8192_bf16_hbm_traffic.md);
# set back to None whenever either kernel changes, until the counters are taken again.
TRAFFIC_BYTES_PER_STEP = 203022849


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--rows", type=int, default=1, help="also time every row of the path (1) or not (0)")
    p.add_argument("--cpu-baseline", type=int, default=1)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (calibrates HBM byte counters) and exit")
    return p.parse_args()


def copy_calibration(mib, reps=4):
    """A plain torch device-to-device copy of `mib` MiB, `reps` times: the
    reference kernel against which FETCH_SIZE / WRITE_SIZE are scaled."""
    import torch
    torch.cuda.set_device(0)
    n = mib << 20
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_scaled_quantization_reduce_amd as fq
    import workloads

    torch.cuda.set_device(0)
    dev = "cuda"
    stream = torch.cuda.current_stream()
    E4, E5 = fq.E4M3FN, fq.E5M2

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ------------------------------------------------ headline: delayed ----
    T = 32
    rows, cols = 8192, 8192
    n = rows * cols
    t0 = time.time()
    host_inputs = workloads.parallel_map(workloads.delayed_step, range(T), workers=16)
    xs = [to_dev(h) for h in host_inputs]
    print("# inputs ready in %.1fs" % (time.time() - t0), file=sys.stderr, flush=True)
    # eight output buffers (512 MiB) in rotation, so that the 256 MB
    # last-level cache cannot hold a step's codes until they are overwritten
    NQ = 8
    qbufs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(NQ)]
    qsi = [torch.empty(1, device=dev) for _ in range(NQ)]
    am = torch.empty(1, device=dev)
    hist = torch.zeros((16, 1), device=dev)
    sc = torch.ones(1, device=dev)
    si = torch.ones(1, device=dev)

    def step(t):
        fmt = E4 if t % 2 == 0 else E5
        fmt_next = E4 if (t + 1) % 2 == 0 else E5
        # cast with the stored scale + fused amax (one kernel), then the
        # partial fold and ring update (one one-block kernel)
        fq.fp8_quantize_delayed(xs[t % T], fmt, hist, 0, t, fmt_next, 0, fq.ALGO_MAX, sc, si, qbufs[t % NQ],
                                qsi[t % NQ], am, stream=stream)

    t = 0
    for _ in range(args.warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()
    # Only two events bracket the timed region: an event between launches
    # costs the GPU several microseconds per step on its own.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(t)
        t += 1
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    bytes_per_step = 3 * n
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    # one step is one launch of the entry point (its two kernels back to back)
    achieved = value

    result = {
        "metric": "quantize GB/s (% HBM peak); scaled FP8 GEMM TFLOPS (% MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->fp8 (fp32 scale arithmetic)",
        "data": "synthetic (seeded numpy generators, resident in HBM)",
        "config": {"workload": "delayed scaling, 32 steps of 8192x8192 bf16, E4M3FN/E5M2 alternating, "
                               "amax history 16 (max), fused input amax",
                   "tensor": [rows, cols], "history_len": 16, "distinct_inputs": T, "distinct_outputs": NQ,
                   "bytes_per_step": bytes_per_step, "host_wall_s": round(wall, 4)},
        "roofline": {"kernel": "fp8_quantize_delayed: cast_kernel (fused amax) + delayed_kernel",
                     "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": TRAFFIC_BYTES_PER_STEP, "kernel_avg_us": round(ms_per_step * 1e3, 3),
                     "algorithmic_bytes_per_launch": bytes_per_step},
    }

    # -------------------------------------------------------- every row ----
    if args.rows:
        result["rows"] = time_rows(fq, torch, np, workloads, to_dev, xs, stream)

    # ------------------------------------------------------ CPU baseline ----
    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, host_inputs, args.cpu_seconds)

    print(json.dumps(result), flush=True)


# Seconds of untimed launches before each row is timed.  The GPU's clocks
# take tens of milliseconds of sustained matrix work to settle: measured on
# the MI355X, the 8192^3 per-tensor GEMM averages 433 us over its first 30
# launches and 380 us once it has run for ~80 ms, while the memory-bound rows
# do not move.  Every row is timed in that steady state.
WARM_S = 0.15


def _time(torch, stream, fn, reps, rotate=1):
    """Average ms of fn(i) over reps launches, HIP events on `stream`, after
    WARM_S seconds of the same launches."""
    i, t0 = 0, time.perf_counter()
    while True:
        fn(i % rotate)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARM_S:
                break
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        fn(i % rotate)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_rows(fq, torch, np, workloads, to_dev, xs, stream):
    dev = "cuda"
    out = {}
    n = xs[0].numel()
    E4, E5 = fq.E4M3FN, fq.E5M2
    am = torch.empty(1, device=dev)
    si = torch.empty(1, device=dev)
    # outputs rotate over sets totalling at least 512 MiB, like the inputs, so
    # that the last-level cache cannot absorb the writes
    qs8 = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(8)]

    def gbs(nbytes, ms):
        g = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 5), "GB/s": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": int(nbytes)}

    # a1 amax over bf16 8192^2 (2 B/elem)
    ms = _time(torch, stream, lambda i: fq.fp8_amax(xs[i], am, stream=stream), 20, rotate=len(xs))
    out["amax_bf16_8192x8192"] = gbs(2 * n, ms)

    # a1+a2+a3 current scaling: amax pass + cast pass (5 B/elem)
    def current(i):
        fq.fp8_amax(xs[i], am, stream=stream)
        fq.fp8_quantize_tensor(xs[i], E4, qs8[i % 8], amax_in=am, margin=0, scale_inv_out=si, stream=stream)
    ms = _time(torch, stream, current, 20, rotate=len(xs))
    out["current_scaling_amax+cast_bf16_8192x8192"] = gbs(5 * n, ms)

    # a4 dequantize 8192^2 codes -> fp32 (1 + 4 B/elem)
    ys = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2)]
    for c in qs8:
        c.random_(0, 256)
    ms = _time(torch, stream, lambda i: fq.fp8_dequantize(qs8[i], E4, si, ys[i % 2], stream=stream), 20, rotate=8)
    out["dequantize_8192x8192_to_fp32"] = gbs(5 * n, ms)

    # a7 rowwise + columnwise per-tensor cast 8192^2 bf16 (2 + 1 + 1 B/elem)
    qr = [q.view(8192, 8192) for q in qs8[:4]]
    qc = [q.view(8192, 8192) for q in qs8[4:]]
    sc1 = torch.full((1,), 0.01, device=dev)
    x2 = [x.view(8192, 8192) for x in xs]
    ms = _time(torch, stream, lambda i: fq.fp8_quantize_rowwise_colwise(
        x2[i], E4, q_row=qr[i % 4], q_col=qc[i % 4], scale_inv_in=sc1, stream=stream), 20, rotate=len(xs))
    out["rowwise_colwise_bf16_8192x8192"] = gbs(4 * n, ms)

    # a8 block quantization of the 7168x4096 weight (128x128) and the
    # 4096x7168 activation (1x128), both with their columnwise copies
    W = torch.randn((7168, 4096), device=dev, generator=torch.Generator(device=dev).manual_seed(1)) * 0.02
    Ws = [(W * (1 + 0.01 * k)).to(torch.bfloat16) for k in range(10)]
    qw = [torch.empty((7168, 4096), dtype=torch.uint8, device=dev) for _ in range(10)]
    qwt = [torch.empty((4096, 7168), dtype=torch.uint8, device=dev) for _ in range(10)]
    sw, swt = torch.empty((56, 32), device=dev), torch.empty((32, 56), device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_quantize_block(Ws[i], E4, 128, qw[i], sw, qwt[i], swt, stream=stream),
               20, rotate=len(Ws))
    nW = 7168 * 4096
    out["block128x128_bf16_7168x4096_with_colwise"] = gbs(4 * nW + 2 * 4 * (nW // 16384), ms)
    X = torch.randn((4096, 7168), device=dev, generator=torch.Generator(device=dev).manual_seed(2))
    Xs = [(X * (1 + 0.01 * k)).to(torch.bfloat16) for k in range(10)]
    qx = [q.view(4096, 7168) for q in qw]
    qxt = [q.view(7168, 4096) for q in qwt]
    sx, sxt = torch.empty((4096, 56), device=dev), torch.empty((7168, 32), device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_quantize_block(Xs[i], E4, 1, qx[i], sx, qxt[i], sxt, stream=stream),
               20, rotate=len(Xs))
    out["block1x128_bf16_4096x7168_with_colwise"] = gbs(4 * nW + 4 * (nW // 128) * 2, ms)
    # next: MXFP8 quantization of 8192^2 bf16 with the columnwise copy
    # (2 + 1 + 1 B/elem + 2 scale bytes per 32 elements)
    sm = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
    smt = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
    ms = _time(torch, stream, lambda i: fq.fp8_quantize_mx(x2[i], E4, qr[i % 4], sm[i % 4], qc[i % 4], smt[i % 4],
                                                           stream=stream), 20, rotate=len(xs))
    out["mxfp8_bf16_8192x8192_with_colwise"] = gbs(4 * n + 2 * n // 32, ms)

    # next: per-direction quantization of 8192^2 bf16, E4M3 rows and E5M2
    # columns from the dequantized rows, current scaling per direction
    # (2 + 1 + 1 B/elem)
    fq.fp8_amax(x2[0], am, stream=stream)
    rsi, csi = torch.empty(1, device=dev), torch.empty(1, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_quantize_hybrid(
        x2[i], E4, E5, fq.COLSRC_ROWWISE_DEQUANTIZED, q_row=qr[i % 4], q_col=qc[i % 4], amax_in=am,
        row_scale_inv_out=rsi, col_scale_inv_out=csi, stream=stream), 20, rotate=len(xs))
    out["hybrid_e4m3_rows_e5m2_cols_dequantized_bf16_8192x8192"] = gbs(4 * n, ms)

    # next: cast statistics (overflow / underflow counts) of 8192^2 bf16
    # under a given scale (2 B/elem read)
    st = torch.empty(4, dtype=torch.int64, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_cast_stats(xs[i], E4, sc1, st, stream=stream), 20, rotate=len(xs))
    out["cast_stats_bf16_8192x8192"] = gbs(2 * n, ms)
    # next: the same counts fused into the cast (given scale, E4M3 codes):
    # 2 B read + 1 B written per element, against 3 B + 2 B for a cast
    # followed by the separate statistics pass
    ms = _time(torch, stream, lambda i: fq.fp8_quantize_tensor_stats(xs[i], E4, qs8[i % 8], st, scale_inv_in=sc1,
                                                                      stream=stream), 20, rotate=len(xs))
    out["cast_with_fused_stats_bf16_8192x8192"] = gbs(3 * n, ms)

    # next: error-feedback quantization of a 64 Mi-element bf16 gradient to
    # E5M2 with its fp32 residual updated in place (2 + 4 + 1 + 4 B/elem)
    del ys
    res = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2)]
    s_ef = torch.full((1,), 2.0 ** -16, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_quantize_error_feedback(xs[i], res[i % 2], E5, s_ef, qs8[i % 8], am,
                                                                       stream=stream), 20, rotate=len(xs))
    out["error_feedback_bf16_to_e5m2_64Mi"] = gbs(11 * n, ms)
    del Ws, Xs, W, X, qw, qwt, qx, qxt, qs8, qr, qc, sm, smt, res

    def tflops(flop, ms):
        tf = flop / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
                "flop": int(flop)}

    # GEMM operands are codes of Gaussian data quantized by the library's own
    # per-tensor cast (the codes a GEMM consumes in practice: random signs,
    # exponents clustered below the format maximum)
    g = torch.Generator(device=dev).manual_seed(3)

    def codes(shape, fmt):
        x = torch.randn(shape, device=dev, generator=g).to(torch.bfloat16)
        c = torch.empty(shape, dtype=torch.uint8, device=dev)
        a = torch.empty(1, device=dev)
        fq.fp8_amax(x, a, stream=stream)
        fq.fp8_quantize_tensor(x, fmt, c, amax_in=a, margin=0, stream=stream)
        del x
        return c

    # a9 per-tensor GEMM 8192^3 E4M3 x E4M3 -> bf16 with output amax
    A = codes((8192, 8192), E4)
    B = codes((8192, 8192), E4)
    C = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    s1 = torch.full((1,), 1e-3, device=dev)
    cam = torch.empty(1, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_scaled_gemm(A, E4, s1, B, E4, s1, fq.PER_TENSOR, C, cam,
                                                            stream=stream), 30)
    out["gemm_per_tensor_e4m3_8192x8192x8192"] = tflops(2 * 8192 ** 3, ms)
    del A, B, C

    # a10 block-scaled GEMMs of the MLP block: fprop 4096x14336x4096 (E4M3 x
    # E4M3) and dgrad 4096x4096x14336 (E5M2 x E4M3)
    Xq = codes((4096, 4096), E4)
    Wq = codes((14336, 4096), E4)
    sx = torch.rand((4096, 32), device=dev, generator=g) + 0.5
    sw = torch.rand((112, 32), device=dev, generator=g) + 0.5
    Y = torch.empty((4096, 14336), dtype=torch.bfloat16, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_scaled_gemm(Xq, E4, sx, Wq, E4, sw, fq.BLOCK_1x128_128x128, Y, cam,
                                                            stream=stream), 30)
    out["gemm_block_fprop_4096x14336x4096"] = tflops(2 * 4096 * 14336 * 4096, ms)
    dYq = codes((4096, 14336), E5)
    Wtq = codes((4096, 14336), E4)
    sdy = torch.rand((4096, 112), device=dev, generator=g) + 0.5
    swt = torch.rand((32, 112), device=dev, generator=g) + 0.5
    dX = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_scaled_gemm(dYq, E5, sdy, Wtq, E4, swt, fq.BLOCK_1x128_128x128, dX,
                                                            cam, stream=stream), 30)
    out["gemm_block_dgrad_4096x4096x14336"] = tflops(2 * 4096 * 4096 * 14336, ms)
    del dYq, Wtq, dX

    # next: the MLP's first projection with its epilogue fused, per-tensor
    # E4M3 x E4M3, H = GELU(X W^T + b) cast to E4M3 codes with a given output
    # scale and the pre-cast amax; beside it the same GEMM with a plain bf16
    # output (the difference is the epilogue's cost)
    bias = torch.randn(14336, device=dev, generator=g) * 0.5
    s_h = torch.full((1,), 6.0 / 448, device=dev)
    H = torch.empty((4096, 14336), dtype=torch.uint8, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_scaled_gemm(Xq, E4, s1, Wq, E4, s1, fq.PER_TENSOR, Y, cam,
                                                            stream=stream), 30)
    out["gemm_per_tensor_fc1_4096x14336x4096_bf16"] = tflops(2 * 4096 * 14336 * 4096, ms)
    ms = _time(torch, stream, lambda i: fq.fp8_scaled_gemm_fused(Xq, E4, s1, Wq, E4, s1, fq.PER_TENSOR, H, bias=bias,
                                                                  act=fq.ACT_GELU, out_fmt=E4, c_scale_inv=s_h,
                                                                  amax_out=cam, stream=stream), 30)
    out["gemm_fused_bias_gelu_e4m3out_4096x14336x4096"] = tflops(2 * 4096 * 14336 * 4096, ms)
    del Xq, Wq, Y, H, bias

    # next: weight gradient dW = dY^T X, fp32 out, both operands the
    # token-contiguous (columnwise) copies with 1x128 scales along the tokens
    dYt = codes((14336, 4096), E5)
    Xt = codes((4096, 4096), E4)
    sdyt = torch.rand((14336, 32), device=dev, generator=g) + 0.5
    sxt = torch.rand((4096, 32), device=dev, generator=g) + 0.5
    dW = torch.empty((14336, 4096), dtype=torch.float32, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_scaled_gemm(dYt, E5, sdyt, Xt, E4, sxt, fq.BLOCK_1x128_1x128, dW,
                                                            cam, stream=stream), 30)
    out["gemm_block_wgrad_14336x4096x4096_fp32out"] = tflops(2 * 14336 * 4096 * 4096, ms)
    del dYt, Xt, dW

    # next: MXFP8 GEMM 8192^3 (E8M0 scales per 32 along K, applied by the
    # matrix instruction), operands from the library's MXFP8 quantization
    def mx_codes(shape):
        x = torch.randn(shape, device=dev, generator=g).to(torch.bfloat16)
        c = torch.empty(shape, dtype=torch.uint8, device=dev)
        e = torch.empty((shape[0], shape[1] // 32), dtype=torch.uint8, device=dev)
        fq.fp8_quantize_mx(x, E4, c, e, stream=stream)
        del x
        return c, e

    Am, sAm = mx_codes((8192, 8192))
    Bm, sBm = mx_codes((8192, 8192))
    Cm = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    ms = _time(torch, stream, lambda i: fq.fp8_scaled_gemm(Am, E4, sAm, Bm, E4, sBm, fq.MXFP8, Cm, cam,
                                                            stream=stream), 30)
    out["gemm_mxfp8_e4m3_8192x8192x8192"] = tflops(2 * 8192 ** 3, ms)
    return out


def cpu_baseline(np, host_inputs, seconds):
    """The oracle's delayed-scaling schedule on the host: the 32 steps, each
    pass from a fresh ring, repeated until `seconds` of work have been done
    (whole steps; at least one)."""
    import oracle

    T = len(host_inputs)
    done = 0
    t0 = time.perf_counter()
    while True:
        t = done % T
        if t == 0:
            hist = np.zeros((16, 1), np.float32)
            sc, si = np.ones(1, np.float32), np.ones(1, np.float32)
        x = host_inputs[t]
        fmt = oracle.E4M3FN if t % 2 == 0 else oracle.E5M2
        fmt_next = oracle.E4M3FN if (t + 1) % 2 == 0 else oracle.E5M2
        r = oracle.quantize_tensor(x, fmt, scale_inv_in=si[0])
        oracle.delayed_update(hist, 0, r["amax"], t, fmt_next, 0, oracle.ALGO_MAX, sc, si)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    nbytes = 3 * host_inputs[0].size * done
    return {"value": round(nbytes / el / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d delayed-scaling steps (the %d-step schedule of 8192x8192 bf16 tensors, repeated from a "
                      "fresh ring; cast with fused amax + ring update each), %.1f s" % (done, T, el)}


if __name__ == "__main__":
    main()
