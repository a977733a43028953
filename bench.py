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
the stream they run on.  One step is one call of the fused entry point, a
single launch (the casting blocks and the finishing block that folds their
amax partials and updates the ring), so the roofline object uses that same
per-step duration.

Every other row of the hot path (the per-tensor fp32 1024x1024 current-scaling
workload, amax, current scaling, dequantize, rowwise + columnwise, 128x128
and 1x128 block quantization, per-tensor and block-scaled GEMMs, and the next
rows) is timed at its own workload size under "rows": the median and the
10th / 90th percentiles of 50 samples, each sample the mean of a few
back-to-back launches between two events, taken after 150 ms of untimed
launches of the same call.  Memory-bound rows report GB/s against the 8 TB/s
peak and against a device copy measured in the same run; GEMM rows report
TFLOP/s against the 5.0 PFLOP/s FP8 peak and against that peak scaled to
the graphics clock the row runs at ("sclk": measured on the device by the
library's clock monitor, which shares CUs with an untimed batch of the same
launches right after the timed samples).  Each row carries the CPU oracle's
rate on the same workload ("cpu"), a baseline only.

The CPU oracle's delayed-scaling schedule is the headline's "cpu_baseline".
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
MFMA_PEAK_SCLK_MHZ = 2400.0  # the clock the 5.0 PFLOP/s figure assumes (256 CUs x 8192 FP8 flop/clk)
# HBM bytes of one delayed step (the cast kernel with its finishing block),
# from the FETCH_SIZE and WRITE_SIZE counters scaled by the factors a plain
# copy gives (profiles/hbm_traffic_bench_kernels.md); None whenever the kernel
# has changed since the counters were taken.
TRAFFIC_BYTES_PER_STEP = 201781495

# Seconds of untimed launches before each row is timed.  The GPU's clocks
# take tens of milliseconds of sustained matrix work to settle: measured on
# the MI355X, the 8192^3 per-tensor GEMM averages 433 us over its first 30
# launches and 380 us once it has run for ~80 ms, while the memory-bound rows
# do not move.  Every row is timed in that steady state.
WARM_S = 0.15
SAMPLES = 50


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--rows", type=int, default=1, help="also time every row of the path (1) or not (0)")
    p.add_argument("--only", default="", help="comma-separated row names: time only these rows")
    p.add_argument("--headline", type=int, default=1, help="time the headline delayed-scaling steps (1) or not (0)")
    p.add_argument("--clock", type=int, default=1,
                   help="measure each row's graphics clock with the clock monitor (1) or not (0: for counter "
                        "collection, which runs kernels one at a time, so the monitor would only time out)")
    p.add_argument("--cpu-baseline", type=int, default=1)
    p.add_argument("--cpu-seconds", type=float, default=6.0)
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


# ---------------------------------------------------------------- timing ----
def _pct(values, q):
    s = sorted(values)
    pos = (len(s) - 1) * q
    lo = int(pos)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


_SIDE = []
CLOCK = [True]


def measure_clock(torch, fq, fn, rotate, ms_per_launch, target_ms=30.0):
    """Graphics clock (MHz, per XCD) while fn runs back to back: an untimed
    batch of about target_ms of launches on the current stream, measured by the
    library's clock monitor, which runs on a side stream (default priority)
    on CUs it shares with the batch until a stop word, set on the current
    stream behind the batch, ends it.  None when the monitor did not see the
    stop word."""
    if not _SIDE:
        _SIDE.append(torch.cuda.Stream())
    out = torch.zeros(3 * fq.CLOCK_BLOCKS + 1, dtype=torch.int64, device="cuda")
    stop = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    fq.fp8q_clock_monitor(out, stop, stream=_SIDE[0])
    for i in range(max(8, int(target_ms / max(ms_per_launch, 1e-3)))):
        fn(i % rotate)
    stop.fill_(1)
    torch.cuda.synchronize()
    mhz = fq.clock_mhz(out.cpu().tolist())
    if not mhz:
        return None
    v = list(mhz.values())
    return {"mean_mhz": round(sum(v) / len(v), 1), "min_mhz": round(min(v), 1), "max_mhz": round(max(v), 1),
            "xcds": len(v)}


def time_launches(torch, stream, fn, per_sample, rotate=1, samples=SAMPLES, fq=None):
    """ms per launch of fn(i): after WARM_S seconds of untimed launches,
    `samples` samples of `per_sample` back-to-back launches, each sample
    between two events on `stream`.  Returns median, p10 and p90, and (given
    the library module fq) the graphics clock of a further untimed batch."""
    i, t0 = 0, time.perf_counter()
    while True:
        fn(i % rotate)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARM_S:
                break
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
    ev[0].record(stream)
    for k in range(samples):
        for _ in range(per_sample):
            fn(i % rotate)
            i += 1
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[k].elapsed_time(ev[k + 1]) / per_sample for k in range(samples)]
    r = {"ms": round(_pct(ms, 0.5), 5), "ms_p10": round(_pct(ms, 0.1), 5), "ms_p90": round(_pct(ms, 0.9), 5),
         "samples": samples, "launches_per_sample": per_sample}
    if fq is not None and CLOCK[0]:
        r["sclk"] = measure_clock(torch, fq, lambda j: fn((i + j) % rotate), rotate, r["ms"])
    return r


def cpu_rate(fn, units, unit, budget_s=3.0, reps=3):
    """Median seconds of fn() over up to `reps` runs within `budget_s` (at
    least one), as `units` per second."""
    import oracle
    times = []
    t_all = time.perf_counter()
    while len(times) < reps:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s:
            break
    med = _pct(times, 0.5)
    return {"value": round(units / med, 3), "unit": unit, "seconds": round(med, 4), "runs": len(times),
            "cores": oracle.num_threads(), "kind": "oracle"}


def blas_threads():
    try:
        import threadpoolctl
        return max(i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    CLOCK[0] = bool(args.clock)
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
    result = {
        "metric": "quantize GB/s (% HBM peak); scaled FP8 GEMM TFLOPS (% MFMA peak)",
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->fp8 (fp32 scale arithmetic)",
        "data": "synthetic (seeded numpy generators, resident in HBM)",
    }
    if args.headline:
        result.update(headline(args, fq, torch, xs, stream, n))

    # -------------------------------------------------------- every row ----
    only = set(x for x in args.only.split(",") if x)
    if args.rows:
        out, ceiling = time_rows(fq, torch, np, workloads, to_dev, xs, stream, only, args.cpu_baseline)
        result["rows"] = out
        result["copy_ceiling"] = ceiling

    # ------------------------------------------------------ CPU baseline ----
    if args.cpu_baseline and args.headline:
        result["cpu_baseline"] = cpu_baseline(np, host_inputs, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def headline(args, fq, torch, xs, stream, n):
    dev = "cuda"
    E4, E5 = fq.E4M3FN, fq.E5M2
    T = len(xs)
    rows, cols = xs[0].shape
    # eight output buffers (512 MiB) in rotation, so that the 256 MB
    # last-level cache cannot hold a step's codes until they are overwritten
    NQ = 8
    qbufs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(NQ)]
    qsi = [torch.empty(1, device=dev) for _ in range(NQ)]
    am = torch.empty(1, device=dev)
    hist = torch.zeros((16, 1), device=dev)
    sc = torch.ones(1, device=dev)
    si = torch.ones(1, device=dev)
    state = {"t": 0}

    def step(_=None):
        t = state["t"]
        fmt = E4 if t % 2 == 0 else E5
        fmt_next = E4 if (t + 1) % 2 == 0 else E5
        # cast with the stored scale + fused amax (one kernel), then the
        # partial fold and ring update (one one-block kernel)
        fq.fp8_quantize_delayed(xs[t % T], fmt, hist, 0, t, fmt_next, 0, fq.ALGO_MAX, sc, si, qbufs[t % NQ],
                                qsi[t % NQ], am, stream=stream)
        state["t"] = t + 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Only two events bracket the timed region: an event between launches
    # costs the GPU several microseconds per step on its own.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    bytes_per_step = 3 * n
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    # the spread of the step time: 50 samples of 8 steps each, after the
    # timed region (the state machine just continues)
    spread = time_launches(torch, stream, step, 8, fq=fq)
    return {
        "value": round(value, 1),
        "ms_per_step": round(ms_per_step, 5),
        "config": {"workload": "delayed scaling, 32 steps of 8192x8192 bf16, E4M3FN/E5M2 alternating, "
                               "amax history 16 (max), fused input amax",
                   "tensor": [rows, cols], "history_len": 16, "distinct_inputs": T, "distinct_outputs": NQ,
                   "bytes_per_step": bytes_per_step, "host_wall_s": round(wall, 4),
                   "step_ms_p10_p50_p90": [spread["ms_p10"], spread["ms"], spread["ms_p90"]],
                   "sclk": spread.get("sclk")},
        "roofline": {"kernel": "fp8_quantize_delayed: cast_kernel (fused amax, finishing block updates the ring)",
                     "bound": "hbm", "achieved": round(value, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": TRAFFIC_BYTES_PER_STEP, "kernel_avg_us": round(ms_per_step * 1e3, 3),
                     "algorithmic_bytes_per_launch": bytes_per_step},
    }


def time_rows(fq, torch, np, workloads, to_dev, xs, stream, only, with_cpu):
    """Every row of the path at its own workload.  Returns (rows, copy ceiling)."""
    import oracle
    dev = "cuda"
    out = {}
    n = xs[0].numel()
    E4, E5 = fq.E4M3FN, fq.E5M2
    am = torch.empty(1, device=dev)
    si = torch.empty(1, device=dev)

    def want(name):
        return not only or name in only

    def timed(fn, per_sample, rotate=1):
        # every row also reports the graphics clock of an untimed batch
        return time_launches(torch, stream, fn, per_sample, rotate, fq=fq)

    # the device copy ceiling of this run: torch's copy of 128 MiB buffers,
    # eight pairs in rotation (2 GiB), read + written bytes per second
    cp_src = [torch.empty(128 << 20, dtype=torch.uint8, device=dev) for _ in range(8)]
    cp_dst = [torch.empty(128 << 20, dtype=torch.uint8, device=dev) for _ in range(8)]
    r = time_launches(torch, stream, lambda i: cp_dst[i].copy_(cp_src[i]), 16, rotate=8)
    ceiling = {"GB/s": round(2 * (128 << 20) / (r["ms"] * 1e-3) / 1e9, 1), "ms": r["ms"],
               "method": "torch device copy of 128 MiB buffers, 8 pairs in rotation, median of 50 samples x 16"}
    del cp_src, cp_dst

    def hbm(name, nbytes, t, cpu=None, note=None):
        g = nbytes / (t["ms"] * 1e-3) / 1e9
        row = dict(t)
        row.update({"GB/s": round(g, 1), "frac_hbm": round(g / HBM_PEAK_GBS, 4),
                    "frac_copy_ceiling": round(g / ceiling["GB/s"], 4), "algorithmic_bytes": int(nbytes)})
        if note:
            row["note"] = note
        if cpu is not None:
            row["cpu"] = cpu
        out[name] = row

    def mfma(name, flop, t, cpu=None):
        tf = flop / (t["ms"] * 1e-3) / 1e12
        row = dict(t)
        row.update({"TFLOP/s": round(tf, 1), "frac_mfma": round(tf / FP8_MFMA_PEAK_TFLOPS, 4), "flop": int(flop)})
        if t.get("sclk"):
            # the FP8 peak scales with the graphics clock the row ran at
            peak = FP8_MFMA_PEAK_TFLOPS * t["sclk"]["mean_mhz"] / MFMA_PEAK_SCLK_MHZ
            row["mfma_peak_at_sclk_tflops"] = round(peak, 1)
            row["frac_mfma_at_sclk"] = round(tf / peak, 4)
        if cpu is not None:
            row["cpu"] = cpu
        out[name] = row

    def cpu(fn, units, unit):
        return cpu_rate(fn, units, unit) if with_cpu else None

    hx = None  # the first headline input on the host, for the CPU rows

    def host_x():
        nonlocal hx
        if hx is None:
            hx = workloads.delayed_step(0)
        return hx

    # cfg1: per-tensor current scaling of the fp32 1024x1024 tensor
    # (amax, cast with margin 1, dequantize: 4 + 4 + 1 + 1 + 4 B/elem) and the
    # two decode tables; launch-bound, its time is reported
    name = "tensor_fp32_1024x1024_amax_cast_dequant_margin1"
    if want(name):
        x1h = workloads.tensor_fp32()
        x1 = to_dev(x1h)
        q1 = torch.empty(x1.numel(), dtype=torch.uint8, device=dev)
        y1 = torch.empty(x1.numel(), dtype=torch.float32, device=dev)
        s1o = torch.empty(1, device=dev)

        def cfg1(i):
            fq.fp8_amax(x1, am, stream=stream)
            fq.fp8_quantize_tensor(x1, E4, q1, amax_in=am, margin=1, scale_inv_out=s1o, stream=stream)
            fq.fp8_dequantize(q1, E4, s1o, y1, stream=stream)
        t = timed(cfg1, 16)

        def cfg1_cpu():
            r = oracle.quantize_tensor(x1h, oracle.E4M3FN, amax_in=oracle.amax(x1h), margin=1)
            oracle.dequantize(r["q"], oracle.E4M3FN, r["scale_inv"])
        hbm(name, 14 * x1.numel(), t, cpu(cfg1_cpu, 14 * x1.numel() / 1e9, "GB/s"),
            note="three launches (amax + its finish, cast, dequantize); launch-bound, time reported")
        codes = torch.arange(256, dtype=torch.int32, device=dev).to(torch.uint8)
        one = torch.ones(1, device=dev)
        tab = torch.empty(256, device=dev)
        t = timed(lambda i: fq.fp8_dequantize(codes, i % 2, one, tab, stream=stream), 16)
        out["decode_tables_256_codes"] = dict(t, note="dequantize of the 256 codes with scale 1, alternating formats")

    # outputs rotate over sets totalling at least 512 MiB, like the inputs, so
    # that the last-level cache cannot absorb the writes
    qs8 = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(8)]

    # a1 amax over bf16 8192^2 (2 B/elem)
    name = "amax_bf16_8192x8192"
    if want(name):
        t = timed(lambda i: fq.fp8_amax(xs[i], am, stream=stream), 16, rotate=len(xs))
        hbm(name, 2 * n, t, cpu(lambda: oracle.amax(host_x()), 2 * n / 1e9, "GB/s"))

    # a1+a2+a3 current scaling: amax pass + cast pass (5 B/elem)
    name = "current_scaling_amax+cast_bf16_8192x8192"
    if want(name):
        def current(i):
            fq.fp8_amax(xs[i], am, stream=stream)
            fq.fp8_quantize_tensor(xs[i], E4, qs8[i % 8], amax_in=am, margin=0, scale_inv_out=si, stream=stream)
        t = timed(current, 8, rotate=len(xs))
        hbm(name, 5 * n, t, cpu(lambda: oracle.quantize_tensor(host_x(), oracle.E4M3FN, amax_in=oracle.amax(host_x())),
                                5 * n / 1e9, "GB/s"))

    # a3 alone: the cast with a given scale (3 B/elem)
    sc1 = torch.full((1,), 0.01, device=dev)
    name = "cast_given_scale_bf16_8192x8192"
    if want(name):
        t = timed(lambda i: fq.fp8_quantize_tensor(xs[i], E4, qs8[i % 8], scale_inv_in=sc1,
                                                                          stream=stream), 16, rotate=len(xs))
        hbm(name, 3 * n, t, cpu(lambda: oracle.quantize(host_x(), oracle.E4M3FN, np.float32(100.0)), 3 * n / 1e9,
                                "GB/s"))

    # a4 dequantize 8192^2 codes -> fp32 (1 + 4 B/elem)
    name = "dequantize_8192x8192_to_fp32"
    if want(name):
        ys = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2)]
        for c in qs8:
            c.random_(0, 256)
        si.fill_(0.01)
        t = timed(lambda i: fq.fp8_dequantize(qs8[i], E4, si, ys[i % 2], stream=stream), 16,
                          rotate=8)
        hq = np.random.default_rng(0).integers(0, 256, n, dtype=np.uint8)
        hbm(name, 5 * n, t, cpu(lambda: oracle.dequantize(hq, oracle.E4M3FN, np.float32(0.01)), 5 * n / 1e9, "GB/s"))
        del ys, hq

    # a7 rowwise + columnwise per-tensor cast 8192^2 bf16 (2 + 1 + 1 B/elem)
    qr = [q.view(8192, 8192) for q in qs8[:4]]
    qc = [q.view(8192, 8192) for q in qs8[4:]]
    x2 = [x.view(8192, 8192) for x in xs]
    name = "rowwise_colwise_bf16_8192x8192"
    if want(name):
        t = timed(lambda i: fq.fp8_quantize_rowwise_colwise(
            x2[i], E4, q_row=qr[i % 4], q_col=qc[i % 4], scale_inv_in=sc1, stream=stream), 16, rotate=len(xs))
        hbm(name, 4 * n, t, cpu(lambda: oracle.quantize_rowwise_colwise(host_x(), oracle.E4M3FN, np.float32(100.0)),
                                4 * n / 1e9, "GB/s"))

    # a8 block quantization of the 7168x4096 weight (128x128) and the
    # 4096x7168 activation (1x128), both with their columnwise copies; ten
    # input and output sets in rotation
    nW = 7168 * 4096
    name_w, name_x = "block128x128_bf16_7168x4096_with_colwise", "block1x128_bf16_4096x7168_with_colwise"
    if want(name_w) or want(name_x):
        qw = [torch.empty((7168, 4096), dtype=torch.uint8, device=dev) for _ in range(10)]
        qwt = [torch.empty((4096, 7168), dtype=torch.uint8, device=dev) for _ in range(10)]
        if want(name_w):
            W = torch.randn((7168, 4096), device=dev, generator=torch.Generator(device=dev).manual_seed(1)) * 0.02
            Ws = [(W * (1 + 0.01 * k)).to(torch.bfloat16) for k in range(10)]
            del W
            sw, swt = torch.empty((56, 32), device=dev), torch.empty((32, 56), device=dev)
            t = timed(lambda i: fq.fp8_quantize_block(Ws[i], E4, 128, qw[i], sw, qwt[i], swt,
                                                                             stream=stream), 16, rotate=len(Ws))
            hw = workloads.block_weight() if with_cpu else None
            hbm(name_w, 4 * nW + 2 * 4 * (nW // 16384), t,
                cpu(lambda: oracle.quantize_block(hw, oracle.E4M3FN, 128), (4 * nW + 8 * (nW // 16384)) / 1e9, "GB/s"))
            del Ws, hw
        if want(name_x):
            X = torch.randn((4096, 7168), device=dev, generator=torch.Generator(device=dev).manual_seed(2))
            Xs = [(X * (1 + 0.01 * k)).to(torch.bfloat16) for k in range(10)]
            del X
            qx = [q.view(4096, 7168) for q in qw]
            qxt = [q.view(7168, 4096) for q in qwt]
            sx, sxt = torch.empty((4096, 56), device=dev), torch.empty((7168, 32), device=dev)
            t = timed(lambda i: fq.fp8_quantize_block(Xs[i], E4, 1, qx[i], sx, qxt[i], sxt,
                                                                             stream=stream), 16, rotate=len(Xs))
            ha = workloads.block_act() if with_cpu else None
            hbm(name_x, 4 * nW + 4 * (nW // 128) * 2, t,
                cpu(lambda: oracle.quantize_block(ha, oracle.E4M3FN, 1), (4 * nW + 8 * (nW // 128)) / 1e9, "GB/s"))
            del Xs, ha
        del qw, qwt

    # next: MXFP8 quantization of 8192^2 bf16 with the columnwise copy
    # (2 + 1 + 1 B/elem + 2 scale bytes per 32 elements)
    name = "mxfp8_bf16_8192x8192_with_colwise"
    if want(name):
        sm = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
        smt = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
        t = timed(lambda i: fq.fp8_quantize_mx(x2[i], E4, qr[i % 4], sm[i % 4], qc[i % 4],
                                                                      smt[i % 4], stream=stream), 16, rotate=len(xs))

        def mx_cpu():
            oracle.quantize_mx(host_x(), oracle.E4M3FN)
            oracle.quantize_mx_colwise(host_x(), oracle.E4M3FN)
        hbm(name, 4 * n + 2 * n // 32, t, cpu(mx_cpu, (4 * n + 2 * n // 32) / 1e9, "GB/s"))
        del sm, smt

    # next: per-direction quantization of 8192^2 bf16, E4M3 rows and E5M2
    # columns from the dequantized rows, current scaling per direction
    # (2 + 1 + 1 B/elem)
    name = "hybrid_e4m3_rows_e5m2_cols_dequantized_bf16_8192x8192"
    if want(name):
        fq.fp8_amax(x2[0], am, stream=stream)
        rsi, csi = torch.empty(1, device=dev), torch.empty(1, device=dev)
        t = timed(lambda i: fq.fp8_quantize_hybrid(
            x2[i], E4, E5, fq.COLSRC_ROWWISE_DEQUANTIZED, q_row=qr[i % 4], q_col=qc[i % 4], amax_in=am,
            row_scale_inv_out=rsi, col_scale_inv_out=csi, stream=stream), 16, rotate=len(xs))

        def hyb_cpu():
            oracle.quantize_hybrid(host_x(), oracle.E4M3FN, oracle.E5M2, oracle.COLSRC_ROWWISE_DEQUANTIZED,
                                   amax_in=oracle.amax(host_x()))
        hbm(name, 4 * n, t, cpu(hyb_cpu, 4 * n / 1e9, "GB/s"))

    # next: per-direction quantization with MXFP8 sub-quantizers, E4M3
    # forward copy and E5M2 backward copy of 8192^2 bf16 in one pass
    # (2 + 1 + 1 B/elem + 2 scale bytes per 32 elements)
    name = "hybrid_mxfp8_e4m3_rows_e5m2_cols_bf16_8192x8192"
    if want(name):
        sm = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
        smt = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
        t = timed(lambda i: fq.fp8_quantize_hybrid_blockwise(
            x2[i], fq.SUBQ_MXFP8, E4, fq.SUBQ_MXFP8, E5, q_row=qr[i % 4], s_row=sm[i % 4], q_col=qc[i % 4],
            s_col=smt[i % 4], stream=stream), 16, rotate=len(xs))

        def hyb_mx_cpu():
            oracle.quantize_hybrid_blockwise(host_x(), oracle.SUBQ_MXFP8, oracle.E4M3FN, oracle.SUBQ_MXFP8,
                                             oracle.E5M2)
        hbm(name, 4 * n + 2 * n // 32, t, cpu(hyb_mx_cpu, (4 * n + 2 * n // 32) / 1e9, "GB/s"))
        del sm, smt

    # next: the same MXFP8 pair with the columnwise copy taken from the
    # dequantized rowwise values (same bytes)
    name = "hybrid_mxfp8_e4m3_rows_e5m2_cols_dequantized_bf16_8192x8192"
    if want(name):
        sm = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
        smt = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
        t = timed(lambda i: fq.fp8_quantize_hybrid_blockwise(
            x2[i], fq.SUBQ_MXFP8, E4, fq.SUBQ_MXFP8, E5, col_source=fq.COLSRC_ROWWISE_DEQUANTIZED, q_row=qr[i % 4],
            s_row=sm[i % 4], q_col=qc[i % 4], s_col=smt[i % 4], stream=stream), 16, rotate=len(xs))

        def hyb_mxd_cpu():
            oracle.quantize_hybrid_blockwise(host_x(), oracle.SUBQ_MXFP8, oracle.E4M3FN, oracle.SUBQ_MXFP8,
                                             oracle.E5M2, oracle.COLSRC_ROWWISE_DEQUANTIZED)
        hbm(name, 4 * n + 2 * n // 32, t, cpu(hyb_mxd_cpu, (4 * n + 2 * n // 32) / 1e9, "GB/s"))
        del sm, smt

    # next: per-direction quantization with two recipes in one pass: 1x128
    # E4M3 rows (a row-scaled forward copy) and MXFP8 E5M2 columns of 8192^2
    # bf16 (2 + 1 + 1 B/elem + 4 B per 128 and 1 B per 32 elements)
    name = "hybrid_1x128_e4m3_rows_mxfp8_e5m2_cols_bf16_8192x8192"
    if want(name):
        sr = [torch.empty((8192, 64), dtype=torch.float32, device=dev) for _ in range(4)]
        smt = [torch.empty((8192, 256), dtype=torch.uint8, device=dev) for _ in range(4)]
        t = timed(lambda i: fq.fp8_quantize_hybrid_blockwise(
            x2[i], fq.SUBQ_BLOCK_1x128, E4, fq.SUBQ_MXFP8, E5, q_row=qr[i % 4], s_row=sr[i % 4], q_col=qc[i % 4],
            s_col=smt[i % 4], stream=stream), 16, rotate=len(xs))

        def hyb_x_cpu():
            oracle.quantize_hybrid_blockwise(host_x(), oracle.SUBQ_BLOCK_1x128, oracle.E4M3FN, oracle.SUBQ_MXFP8,
                                             oracle.E5M2)
        nb = 4 * n + 4 * n // 128 + n // 32
        hbm(name, nb, t, cpu(hyb_x_cpu, nb / 1e9, "GB/s"))
        del sr, smt

    # next: cast statistics (overflow / underflow counts) of 8192^2 bf16
    # under a given scale (2 B/elem read), alone and fused into the cast
    # (2 B read + 1 B written per element, against 3 B + 2 B for a cast
    # followed by the separate statistics pass)
    st = torch.empty(4, dtype=torch.int64, device=dev)
    name = "cast_stats_bf16_8192x8192"
    if want(name):
        t = timed(lambda i: fq.fp8_cast_stats(xs[i], E4, sc1, st, stream=stream), 16,
                          rotate=len(xs))
        hbm(name, 2 * n, t, cpu(lambda: oracle.cast_stats(host_x(), oracle.E4M3FN, np.float32(0.01)), 2 * n / 1e9,
                                "GB/s"))
    name = "cast_with_fused_stats_bf16_8192x8192"
    if want(name):
        t = timed(lambda i: fq.fp8_quantize_tensor_stats(xs[i], E4, qs8[i % 8], st,
                                                                                scale_inv_in=sc1, stream=stream),
                          16, rotate=len(xs))

        def stats_cpu():
            oracle.quantize(host_x(), oracle.E4M3FN, np.float32(100.0))
            oracle.cast_stats(host_x(), oracle.E4M3FN, np.float32(0.01))
        hbm(name, 3 * n, t, cpu(stats_cpu, 3 * n / 1e9, "GB/s"))

    # next: error-feedback quantization of a 64 Mi-element bf16 gradient to
    # E5M2 with its fp32 residual updated in place (2 + 4 + 1 + 4 B/elem)
    name = "error_feedback_bf16_to_e5m2_64Mi"
    if want(name):
        res = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2)]
        s_ef = torch.full((1,), 2.0 ** -16, device=dev)
        t = timed(lambda i: fq.fp8_quantize_error_feedback(xs[i], res[i % 2], E5, s_ef,
                                                                                  qs8[i % 8], am, stream=stream),
                          8, rotate=len(xs))
        hres = np.zeros(n, np.float32) if with_cpu else None
        hbm(name, 11 * n, t, cpu(lambda: oracle.quantize_error_feedback(host_x().reshape(-1), hres, oracle.E5M2,
                                                                        np.float32(2.0 ** -16)), 11 * n / 1e9, "GB/s"))
        del res, hres
    del qs8, qr, qc

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

    # CPU baseline of the GEMM rows: the oracle's float64 reference (decode,
    # then numpy's BLAS matmul; block modes loop over the 128-wide K slices)
    # on a sample of the output rows; GFLOP/s of that sample
    rng = np.random.default_rng(0)

    def gemm_cpu(M, N, K, fa, fb, mode, rows_sample):
        if not with_cpu:
            return None
        A = rng.integers(0, 0x70, (rows_sample, K), dtype=np.uint8)
        B = rng.integers(0, 0x70, (N, K), dtype=np.uint8)
        if mode == oracle.PER_TENSOR:
            sA, sB = np.float32(1e-3), np.float32(1e-3)
        elif mode == oracle.BLOCK_1x128_128x128:
            sA, sB = np.ones((rows_sample, K // 128), np.float32), np.ones((N // 128, K // 128), np.float32)
        elif mode == oracle.BLOCK_1x128_1x128:
            sA, sB = np.ones((rows_sample, K // 128), np.float32), np.ones((N, K // 128), np.float32)
        else:
            sA, sB = np.full((rows_sample, K // 32), 120, np.uint8), np.full((N, K // 32), 120, np.uint8)
        r = cpu_rate(lambda: oracle.gemm_reference(A, fa, sA, B, fb, sB, mode), 2.0 * rows_sample * N * K / 1e9,
                     "GFLOP/s", budget_s=4.0, reps=2)
        r["cores"] = blas_threads()
        r["sample"] = "%d of %d output rows (float64 reference: decode + BLAS matmul)" % (rows_sample, M)
        return r

    cam = torch.empty(1, device=dev)
    s1 = torch.full((1,), 1e-3, device=dev)

    # a9 per-tensor GEMM 8192^3 E4M3 x E4M3 -> bf16 with output amax
    name = "gemm_per_tensor_e4m3_8192x8192x8192"
    if want(name):
        A = codes((8192, 8192), E4)
        B = codes((8192, 8192), E4)
        C = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
        t = timed(lambda i: fq.fp8_scaled_gemm(A, E4, s1, B, E4, s1, fq.PER_TENSOR, C, cam,
                                                                       stream=stream), 4)
        mfma(name, 2 * 8192 ** 3, t, gemm_cpu(8192, 8192, 8192, oracle.E4M3FN, oracle.E4M3FN, oracle.PER_TENSOR, 512))
        del A, B, C

    # a10 block-scaled GEMMs of the MLP block: fprop 4096x14336x4096 (E4M3 x
    # E4M3) and dgrad 4096x4096x14336 (E5M2 x E4M3)
    Xq = Wq = None
    name = "gemm_block_fprop_4096x14336x4096"
    names_fc1 = ("gemm_per_tensor_fc1_4096x14336x4096_bf16", "gemm_fused_bias_gelu_e4m3out_4096x14336x4096")
    if want(name) or any(want(x) for x in names_fc1):
        Xq = codes((4096, 4096), E4)
        Wq = codes((14336, 4096), E4)
        Y = torch.empty((4096, 14336), dtype=torch.bfloat16, device=dev)
    if want(name):
        sx = torch.rand((4096, 32), device=dev, generator=g) + 0.5
        sw = torch.rand((112, 32), device=dev, generator=g) + 0.5
        t = timed(lambda i: fq.fp8_scaled_gemm(Xq, E4, sx, Wq, E4, sw, fq.BLOCK_1x128_128x128,
                                                                       Y, cam, stream=stream), 4)
        mfma(name, 2 * 4096 * 14336 * 4096, t,
             gemm_cpu(4096, 14336, 4096, oracle.E4M3FN, oracle.E4M3FN, oracle.BLOCK_1x128_128x128, 256))
    # the same fprop on one GPU's share of a tensor-parallel layer: the 8-way
    # column shard of W (N = 1792 = 14336 / 8), 112 tiles of 256x256, fewer
    # than the CUs, so it runs as 224 half tiles
    name = "gemm_block_fprop_tp8_shard_4096x1792x4096"
    if want(name):
        if Xq is None:
            Xq = codes((4096, 4096), E4)
            Wq = codes((14336, 4096), E4)
        sx8 = torch.rand((4096, 32), device=dev, generator=g) + 0.5
        sw8 = torch.rand((14, 32), device=dev, generator=g) + 0.5
        W8 = Wq[:1792]
        Y8 = torch.empty((4096, 1792), dtype=torch.bfloat16, device=dev)
        t = timed(lambda i: fq.fp8_scaled_gemm(Xq, E4, sx8, W8, E4, sw8, fq.BLOCK_1x128_128x128, Y8, cam,
                                               stream=stream), 4)
        mfma(name, 2 * 4096 * 1792 * 4096, t,
             gemm_cpu(4096, 1792, 4096, oracle.E4M3FN, oracle.E4M3FN, oracle.BLOCK_1x128_128x128, 512))
        del Y8
    name = "gemm_block_dgrad_4096x4096x14336"
    if want(name):
        dYq = codes((4096, 14336), E5)
        Wtq = codes((4096, 14336), E4)
        sdy = torch.rand((4096, 112), device=dev, generator=g) + 0.5
        swt = torch.rand((32, 112), device=dev, generator=g) + 0.5
        dX = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
        t = timed(lambda i: fq.fp8_scaled_gemm(dYq, E5, sdy, Wtq, E4, swt,
                                                                       fq.BLOCK_1x128_128x128, dX, cam,
                                                                       stream=stream), 4)
        mfma(name, 2 * 4096 * 4096 * 14336, t,
             gemm_cpu(4096, 4096, 14336, oracle.E5M2, oracle.E4M3FN, oracle.BLOCK_1x128_128x128, 256))
        del dYq, Wtq, dX

    # next: the MLP's first projection with its epilogue fused, per-tensor
    # E4M3 x E4M3, H = GELU(X W^T + b) cast to E4M3 codes with a given output
    # scale and the pre-cast amax; beside it the same GEMM with a plain bf16
    # output (the difference is the epilogue's cost)
    if any(want(x) for x in names_fc1):
        bias = torch.randn(14336, device=dev, generator=g) * 0.5
        s_h = torch.full((1,), 6.0 / 448, device=dev)
        H = torch.empty((4096, 14336), dtype=torch.uint8, device=dev)
        if want(names_fc1[0]):
            t = timed(lambda i: fq.fp8_scaled_gemm(Xq, E4, s1, Wq, E4, s1, fq.PER_TENSOR, Y,
                                                                           cam, stream=stream), 4)
            mfma(names_fc1[0], 2 * 4096 * 14336 * 4096, t)
        if want(names_fc1[1]):
            t = timed(lambda i: fq.fp8_scaled_gemm_fused(
                Xq, E4, s1, Wq, E4, s1, fq.PER_TENSOR, H, bias=bias, act=fq.ACT_GELU, out_fmt=E4, c_scale_inv=s_h,
                amax_out=cam, stream=stream), 4)
            mfma(names_fc1[1], 2 * 4096 * 14336 * 4096, t)
        del H, bias
    del Xq, Wq

    # next: weight gradient dW = dY^T X, fp32 out, both operands the
    # token-contiguous (columnwise) copies with 1x128 scales along the tokens
    name = "gemm_block_wgrad_14336x4096x4096_fp32out"
    if want(name):
        dYt = codes((14336, 4096), E5)
        Xt = codes((4096, 4096), E4)
        sdyt = torch.rand((14336, 32), device=dev, generator=g) + 0.5
        sxt = torch.rand((4096, 32), device=dev, generator=g) + 0.5
        dW = torch.empty((14336, 4096), dtype=torch.float32, device=dev)
        t = timed(lambda i: fq.fp8_scaled_gemm(dYt, E5, sdyt, Xt, E4, sxt,
                                                                       fq.BLOCK_1x128_1x128, dW, cam, stream=stream),
                          4)
        mfma(name, 2 * 14336 * 4096 * 4096, t,
             gemm_cpu(14336, 4096, 4096, oracle.E5M2, oracle.E4M3FN, oracle.BLOCK_1x128_1x128, 512))
        del dYt, Xt, dW

    # next: MXFP8 GEMM 8192^3 (E8M0 scales per 32 along K, applied by the
    # matrix instruction), operands from the library's MXFP8 quantization
    name = "gemm_mxfp8_e4m3_8192x8192x8192"
    if want(name):
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
        t = timed(lambda i: fq.fp8_scaled_gemm(Am, E4, sAm, Bm, E4, sBm, fq.MXFP8, Cm, cam,
                                                                       stream=stream), 4)
        mfma(name, 2 * 8192 ** 3, t, gemm_cpu(8192, 8192, 8192, oracle.E4M3FN, oracle.E4M3FN, oracle.MXFP8, 512))
    return out, ceiling


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
            "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": "%d delayed-scaling steps (the %d-step schedule of 8192x8192 bf16 tensors, repeated from a "
                      "fresh ring; cast with fused amax + ring update each), %.1f s" % (done, T, el)}


if __name__ == "__main__":
    main()
