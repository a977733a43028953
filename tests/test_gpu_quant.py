"""GPU parity of the quantization kernels against the CPU oracle.

Codes, scales, amaxes and ring state must be bit-identical to the oracle on
the same seeded inputs (NaN scalars compared as a class).  Every output buffer
is pre-filled with a sentinel, so a byte the kernel fails to write shows up as
a mismatch.  All calls go through the C ABI (ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import empty_codes, empty_f32, first_mismatches, f32_bits, host, same_f32, scalar, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2


def _gpu_amax(x: np.ndarray) -> np.float32:
    xd = to_dev(x)
    out = scalar(-1.0)
    fq.fp8_amax(xd, out)
    return host(out)[0]


# ------------------------------------------------------------------ amax ----
@pytest.mark.parametrize("n", [0, 1, 7, 15, 16, 17, 4095, 1000003])
def test_amax_ragged_sizes(n):
    rng = np.random.default_rng(n)
    xf = (rng.standard_normal(n) * 3).astype(np.float32)
    xb = workloads.to_bf16_bits(rng.standard_normal(n) * 3)
    for x in (xf, xb):
        got = _gpu_amax(x)
        assert f32_bits(got) == f32_bits(oracle.amax(x)), (n, got, oracle.amax(x))


def test_amax_specials():
    x = workloads.tensor_fp32(64, 64, seed=4)
    for pos, v in ((0, np.inf), (4095, -np.inf), (77, np.float32(np.nan)), (5, -np.float32(np.nan))):
        y = x.copy().ravel()
        y[pos] = v
        assert same_f32(_gpu_amax(y), oracle.amax(y))
        if np.isnan(v):
            assert f32_bits(_gpu_amax(y)) == 0x7FC00000
    yb = workloads.to_bf16_bits(x.astype(np.float64))
    yb.ravel()[100] = 0xFFC1  # negative bf16 NaN
    assert f32_bits(_gpu_amax(yb)) == 0x7FC00000
    z = np.zeros(1000, np.float32)
    z[3] = -0.0
    assert f32_bits(_gpu_amax(z)) == 0


def test_amax_tensor_fp32_and_full_size_bf16():
    x = workloads.tensor_fp32()
    assert _gpu_amax(x) == np.float32(2000.0)
    xb = workloads.delayed_step(7)  # 8192 x 8192 bf16
    assert f32_bits(_gpu_amax(xb)) == f32_bits(oracle.amax(xb))


def test_amax_streamed_head_and_cached_tail():
    """Inputs of 160 MiB: the amax pass streams the head and loads the last
    128 MiB plainly (kept in the caches for the cast that follows).  The
    maximum is placed in the first element, on both sides of that boundary
    (in units of 16 KiB counted from the start), in the last whole unit and in
    the tail shorter than one 16-byte vector; each case against the oracle."""
    unit_bytes, kept_bytes = 16 << 10, 128 << 20
    rng = np.random.default_rng(44)
    for dtype_bytes, n in ((2, (80 << 20) + 123), (4, (40 << 20) + 5)):
        if dtype_bytes == 2:
            base = workloads.to_bf16_bits(rng.standard_normal(n))
            big = np.uint16(0x4700)    # 32768.0
        else:
            base = rng.standard_normal(n).astype(np.float32)
            big = np.float32(-32768.5)
        per_vec = 16 // dtype_bytes
        units = -(-(n // per_vec) // 1024)
        boundary = (units - kept_bytes // unit_bytes) * (unit_bytes // dtype_bytes)
        xd = to_dev(base)
        for pos in (0, boundary - 1, boundary, n - 200, n - 1):
            x = base.copy()
            x[pos] = big
            xd.copy_(to_dev(x))
            out = scalar(-1.0)
            fq.fp8_amax(xd, out)
            assert f32_bits(host(out)[0]) == f32_bits(oracle.amax(x)), (dtype_bytes, pos)


# ---------------------------------------------------------- per-tensor cast --
def _gpu_quantize(x, fmt, *, amax_in=None, margin=0, scale_inv_in=None, with_amax=False):
    xd = to_dev(x)
    q = empty_codes(x.size)
    si, sc = scalar(-3.0), scalar(-3.0)
    am = scalar(-3.0) if with_amax else None
    kw = dict(margin=margin, scale_inv_out=si, scale_out=sc, amax_out=am)
    if amax_in is not None:
        kw["amax_in"] = scalar(amax_in)
    else:
        kw["scale_inv_in"] = scalar(scale_inv_in)
    fq.fp8_quantize_tensor(xd, fmt, q, **kw)
    return dict(q=host(q).reshape(x.shape), scale_inv=host(si)[0], scale=host(sc)[0],
                amax=host(am)[0] if with_amax else None)


def _check_quantize(x, fmt, **kw):
    got = _gpu_quantize(x, fmt, with_amax=True, **kw)
    want = oracle.quantize_tensor(x, fmt, amax_in=kw.get("amax_in"), margin=kw.get("margin", 0),
                                  scale_inv_in=kw.get("scale_inv_in"))
    assert np.array_equal(got["q"], want["q"]), first_mismatches(got["q"], want["q"])
    assert same_f32(got["scale_inv"], want["scale_inv"]), (got["scale_inv"], want["scale_inv"])
    assert same_f32(got["scale"], want["scale"]), (got["scale"], want["scale"])
    assert same_f32(got["amax"], want["amax"]), (got["amax"], want["amax"])
    return got


def test_tensor_fp32_current_scaling_e4m3_margin1():
    """1024x1024 fp32, N(0,1)*300 with sixteen +-2000 outliers, E4M3FN, margin 1."""
    x = workloads.tensor_fp32()
    a = _gpu_amax(x)
    got = _check_quantize(x, E4, amax_in=a, margin=1)
    assert f32_bits(got["scale_inv"]) == 0x410EDB6E and f32_bits(got["scale"]) == 0x3DE56041


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("n", [1, 15, 16, 33, 12345, 1 << 20])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_cast_current_ragged(fmt, n, dt):
    rng = np.random.default_rng(n + 7 * fmt)
    v = rng.standard_normal(n) * 5
    x = v.astype(np.float32) if dt == "f32" else workloads.to_bf16_bits(v)
    for margin in (0, 1, -2):
        _check_quantize(x, fmt, amax_in=oracle.amax(x), margin=margin)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_cast_given_scale_with_fused_amax(fmt):
    x = workloads.delayed_step(5, 1000, 1031)
    for s in (1.0, 0.0123, 3.5e-5, 977.0):
        _check_quantize(x, fmt, scale_inv_in=s)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_cast_special_values_and_scales(fmt):
    sv = workloads.special_values_f32()
    rng = np.random.default_rng(2)
    x = np.concatenate([sv, -sv, (rng.standard_normal(101) * 1e3).astype(np.float32)])
    for s in (1.0, 0.0, float("inf"), float("nan"), -2.0, 1e-30, 3e38):
        _check_quantize(x, fmt, scale_inv_in=s)
    for a in (0.0, float("inf"), float("nan"), 1e-40, 3e38):
        _check_quantize(x, fmt, amax_in=a, margin=0)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_cast_all_bf16_patterns(fmt):
    """Every bf16 bit pattern at several scales."""
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for s in (1.0, 2.0 ** -7, 2.0 ** 7, 0.31, 7.7, 1e-30):
        _check_quantize(x, fmt, scale_inv_in=s)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_cast_fp32_boundaries_and_random_patterns(fmt):
    """Every midpoint between neighbouring codes and its binary32 neighbours,
    plus 4M random binary32 bit patterns, at scale 1 and 1/3."""
    v = oracle.decode_table(fmt)[: oracle.max_code(fmt) + 1]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    b = np.concatenate([mids, v.astype(np.float32)]).view(np.uint32).astype(np.int64)
    near = np.concatenate([np.clip(b + d, 0, 0x7F7FFFFF) for d in range(-3, 4)]).astype(np.uint32).view(np.float32)
    rng = np.random.default_rng(99)
    rnd = rng.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([near, -near, rnd])
    for s in (1.0, 3.0):
        _check_quantize(x, fmt, scale_inv_in=s)


def test_cast_is_deterministic():
    x = workloads.delayed_step(3, 2048, 2048)
    a = _gpu_quantize(x, E5, scale_inv_in=0.01, with_amax=True)
    b = _gpu_quantize(x, E5, scale_inv_in=0.01, with_amax=True)
    assert np.array_equal(a["q"], b["q"]) and f32_bits(a["amax"]) == f32_bits(b["amax"])


# --------------------------------------------------------------- dequant ----
@pytest.mark.parametrize("fmt", [E4, E5])
def test_decode_tables(fmt):
    """Dequantizing the 256 codes with scale_inv = 1 gives the decode table."""
    codes = np.arange(256, dtype=np.uint8)
    y = empty_f32(256)
    fq.fp8_dequantize(to_dev(codes), fmt, scalar(1.0), y)
    assert same_f32(host(y), oracle.decode_table(fmt).astype(np.float32))


@pytest.mark.parametrize("fmt", [E4, E5])
def test_dequant_parity(fmt):
    rng = np.random.default_rng(3)
    for n in (1, 17, 100003):
        q = rng.integers(0, 256, n).astype(np.uint8)
        for s in (1.0, 8.9285717, 1e-20, -0.5):
            y = empty_f32(n)
            fq.fp8_dequantize(to_dev(q), fmt, scalar(s), y)
            assert same_f32(host(y), oracle.dequantize(q, fmt, s))


def test_tensor_fp32_quantize_dequantize_roundtrip():
    x = workloads.tensor_fp32()
    xd = to_dev(x)
    am, q, si = scalar(), empty_codes(x.size), scalar()
    fq.fp8_amax(xd, am)
    fq.fp8_quantize_tensor(xd, E4, q, amax_in=am, margin=1, scale_inv_out=si)
    y = empty_f32(x.size)
    fq.fp8_dequantize(q, E4, si, y)
    want = oracle.quantize_tensor(x, E4, amax_in=oracle.amax(x), margin=1)
    assert same_f32(host(y).reshape(x.shape), oracle.dequantize(want["q"], E4, want["scale_inv"]))


# --------------------------------------------------------------- delayed ----
def _run_delayed(inputs, L=16, algo=oracle.ALGO_MAX, margin=0, hist_dev=None, sc=None, si=None, t0=0):
    """Drive the delayed-scaling schedule on the GPU: step t quantizes input t
    (E4M3FN for even t, E5M2 for odd t) with the stored scale, records the
    fused amax, and updates one shared ring for the format of step t+1."""
    hist = hist_dev if hist_dev is not None else torch.zeros((L, 1), dtype=torch.float32, device="cuda")
    sc = sc if sc is not None else torch.ones(1, dtype=torch.float32, device="cuda")
    si = si if si is not None else torch.ones(1, dtype=torch.float32, device="cuda")
    out = []
    for i, x in enumerate(inputs):
        t = t0 + i
        fmt = E4 if t % 2 == 0 else E5
        fmt_next = E4 if (t + 1) % 2 == 0 else E5
        xd = to_dev(x)
        q, qsi, am = empty_codes(x.size), scalar(-1.0), scalar(-1.0)
        fq.fp8_quantize_tensor(xd, fmt, q, scale_inv_in=si, scale_inv_out=qsi, amax_out=am)
        fq.fp8_update_scale_delayed(hist, 0, am, t, fmt_next, margin, algo, sc, si)
        out.append(dict(q=host(q).reshape(x.shape), s=host(qsi)[0], amax=host(am)[0], hist=host(hist).copy(),
                        scale=host(sc)[0], scale_inv=host(si)[0]))
    return out, (hist, sc, si)


def _oracle_delayed(inputs, L=16, algo=oracle.ALGO_MAX, margin=0):
    hist = np.zeros((L, 1), np.float32)
    sc, si = np.ones(1, np.float32), np.ones(1, np.float32)
    out = []
    for t, x in enumerate(inputs):
        fmt = E4 if t % 2 == 0 else E5
        fmt_next = E4 if (t + 1) % 2 == 0 else E5
        r = oracle.quantize_tensor(x, fmt, scale_inv_in=si[0])
        oracle.delayed_update(hist, 0, r["amax"], t, fmt_next, margin, algo, sc, si)
        out.append(dict(q=r["q"], s=r["scale_inv"], amax=r["amax"], hist=hist.copy(), scale=sc[0], scale_inv=si[0]))
    return out


def _compare_delayed(got, want):
    for t, (g, w) in enumerate(zip(got, want)):
        assert np.array_equal(g["q"], w["q"]), (t, first_mismatches(g["q"], w["q"]))
        for k in ("s", "amax", "scale", "scale_inv"):
            assert same_f32(g[k], w[k]), (t, k, g[k], w[k])
        assert same_f32(g["hist"], w["hist"]), (t, g["hist"].ravel(), w["hist"].ravel())


@pytest.mark.parametrize("algo", [oracle.ALGO_MAX, oracle.ALGO_MOST_RECENT])
def test_delayed_32_steps_small(algo):
    inputs = [workloads.delayed_step(t, 256, 400) for t in range(32)]
    got, _ = _run_delayed(inputs, algo=algo)
    _compare_delayed(got, _oracle_delayed(inputs, algo=algo))


def _run_delayed_fused(inputs, L=16, algo=oracle.ALGO_MAX, margin=0):
    """The same schedule through the fused one-call step."""
    hist = torch.zeros((L, 1), dtype=torch.float32, device="cuda")
    sc = torch.ones(1, dtype=torch.float32, device="cuda")
    si = torch.ones(1, dtype=torch.float32, device="cuda")
    out = []
    for t, x in enumerate(inputs):
        fmt = E4 if t % 2 == 0 else E5
        fmt_next = E4 if (t + 1) % 2 == 0 else E5
        q, qsi, am = empty_codes(x.size), scalar(-1.0), scalar(-1.0)
        fq.fp8_quantize_delayed(to_dev(x), fmt, hist, 0, t, fmt_next, margin, algo, sc, si, q, qsi, am)
        out.append(dict(q=host(q).reshape(x.shape), s=host(qsi)[0], amax=host(am)[0], hist=host(hist).copy(),
                        scale=host(sc)[0], scale_inv=host(si)[0]))
    return out


@pytest.mark.parametrize("algo", [oracle.ALGO_MAX, oracle.ALGO_MOST_RECENT])
def test_delayed_fused_step_32_steps(algo):
    inputs = [workloads.delayed_step(t, 192, 336) for t in range(32)]
    _compare_delayed(_run_delayed_fused(inputs, algo=algo), _oracle_delayed(inputs, algo=algo))


def test_delayed_fused_step_ragged_and_nan():
    rng = np.random.default_rng(4)
    inputs = [workloads.to_bf16_bits(rng.standard_normal(n) * 3) for n in (1, 17, 1000003, 0, 33)]
    inputs[2][77] = 0x7FC1  # a NaN element: amax NaN, then the ring holds NaN
    _compare_delayed(_run_delayed_fused(inputs, L=4), _oracle_delayed(inputs, L=4))


def test_delayed_resume_matches_straight_run():
    """32 steps straight == 16 steps, state copied to the host and back into
    fresh buffers, then 16 more steps."""
    inputs = [workloads.delayed_step(t, 128, 256) for t in range(32)]
    straight, _ = _run_delayed(inputs)
    first, (h, sc, si) = _run_delayed(inputs[:16])
    h2, sc2, si2 = (torch.from_numpy(host(v).copy()).cuda() for v in (h, sc, si))
    second, _ = _run_delayed(inputs[16:], hist_dev=h2, sc=sc2, si=si2, t0=16)
    for a, b in zip(straight, first + second):
        assert np.array_equal(a["q"], b["q"])
        for k in ("s", "amax", "scale", "scale_inv"):
            assert f32_bits(a[k]) == f32_bits(b[k])


def test_delayed_nan_amax_and_long_history():
    hist = torch.zeros((1000, 3), dtype=torch.float32, device="cuda")
    hist[:, 2] = 5.0
    sc, si = torch.ones(3, device="cuda"), torch.ones(3, device="cuda")
    h_ref = np.zeros((1000, 3), np.float32)
    h_ref[:, 2] = 5.0
    sc_ref, si_ref = np.ones(3, np.float32), np.ones(3, np.float32)
    rng = np.random.default_rng(1)
    vals = list(np.float32(rng.uniform(0, 100, 20))) + [np.float32(np.nan), np.float32(0.0)]
    for t, v in enumerate(vals):
        fq.fp8_update_scale_delayed(hist, 1, scalar(v), t, E5, 3, oracle.ALGO_MAX, sc, si)
        oracle.delayed_update(h_ref, 1, v, t, E5, 3, oracle.ALGO_MAX, sc_ref, si_ref)
        assert same_f32(host(hist), h_ref) and same_f32(host(sc), sc_ref) and same_f32(host(si), si_ref), t


def test_delayed_full_size_32_steps():
    """The full schedule: 32 steps of 8192x8192 bf16, ring of 16, alternating
    E4M3FN / E5M2, one shared ring that wraps at step 16 -- through the two
    calls and through the fused step the benchmark times."""
    inputs = workloads.parallel_map(workloads.delayed_step, range(32))
    want = _oracle_delayed(inputs)
    got, _ = _run_delayed(inputs)
    _compare_delayed(got, want)
    _compare_delayed(_run_delayed_fused(inputs), want)


# ---------------------------------------------------- rowwise + colwise ----
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("shape", [(16, 16), (144, 272), (128, 128), (400, 1040)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rowwise_colwise_parity(fmt, shape, dt):
    rows, cols = shape
    rng = np.random.default_rng(rows + cols)
    v = rng.standard_normal(shape) * 7
    x = v.astype(np.float32) if dt == "f32" else workloads.to_bf16_bits(v)
    xd = to_dev(x)
    a = oracle.amax(x)
    qr, qc = empty_codes((rows, cols)), empty_codes((cols, rows))
    si, sc, am = scalar(), scalar(), scalar(-1.0)
    fq.fp8_quantize_rowwise_colwise(xd, fmt, q_row=qr, q_col=qc, amax_in=scalar(a), margin=1, scale_inv_out=si,
                                    scale_out=sc, amax_out=am)
    s_ref, sc_ref = oracle.current_scale(a, fmt, 1)
    qr_ref, qc_ref = oracle.quantize_rowwise_colwise(x, fmt, sc_ref)
    assert np.array_equal(host(qr), qr_ref), first_mismatches(host(qr), qr_ref)
    assert np.array_equal(host(qc), qc_ref), first_mismatches(host(qc), qc_ref)
    assert same_f32(host(si)[0], s_ref) and same_f32(host(sc)[0], sc_ref) and same_f32(host(am)[0], a)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("s", [0.37, 0.0, np.inf, np.nan, -2.0])
def test_rowwise_colwise_specials_and_edge_scales(dt, s):
    """NaN, infinities and zeros in the input under ordinary and degenerate
    given scales (0 and inf make inf * 0 and 0 * inf products NaN): every
    code, including NaN codes and their signs, equals the oracle's."""
    rows, cols = 144, 272
    v = np.random.default_rng(4).standard_normal((rows, cols)) * 50
    v[3, 5], v[77, 200], v[143, 271], v[10, 10], v[11, 11] = np.nan, np.inf, -np.inf, 0.0, -0.0
    x = v.astype(np.float32) if dt == "f32" else workloads.to_bf16_bits(v)
    qr, qc = empty_codes((rows, cols)), empty_codes((cols, rows))
    fq.fp8_quantize_rowwise_colwise(to_dev(x), E4, q_row=qr, q_col=qc, scale_inv_in=scalar(s))
    qr_ref, qc_ref = oracle.quantize_rowwise_colwise(x, E4, oracle.reciprocal(np.float32(s)))
    assert np.array_equal(host(qr), qr_ref), first_mismatches(host(qr), qr_ref)
    assert np.array_equal(host(qc), qc_ref), first_mismatches(host(qc), qc_ref)


def test_rowwise_colwise_full_size_given_scale():
    x = workloads.delayed_step(9)
    rows, cols = x.shape
    qr, qc = empty_codes((rows, cols)), empty_codes((cols, rows))
    am = scalar(-1.0)
    fq.fp8_quantize_rowwise_colwise(to_dev(x), E5, q_row=qr, q_col=qc, scale_inv_in=scalar(1e-3), amax_out=am)
    qr_ref, qc_ref = oracle.quantize_rowwise_colwise(x, E5, oracle.reciprocal(np.float32(1e-3)))
    assert np.array_equal(host(qr), qr_ref)
    assert np.array_equal(host(qc), qc_ref)
    assert same_f32(host(am)[0], oracle.amax(x))


def test_colwise_only():
    x = workloads.delayed_step(2, 64, 96)
    qc = empty_codes((96, 64))
    fq.fp8_quantize_rowwise_colwise(to_dev(x), E4, q_col=qc, scale_inv_in=scalar(0.002))
    _, qc_ref = oracle.quantize_rowwise_colwise(x, E4, oracle.reciprocal(np.float32(0.002)))
    assert np.array_equal(host(qc), qc_ref)


# ----------------------------------------------------------------- block ----
def _gpu_block(x, fmt, block_rows, colwise=True):
    rows, cols = x.shape
    xd = to_dev(x)
    qr = empty_codes((rows, cols))
    sr = empty_f32((rows // block_rows, cols // 128))
    qc = sc = None
    if colwise:
        qc = empty_codes((cols, rows))
        sc = empty_f32((cols // 128, rows // 128) if block_rows == 128 else (cols, rows // 128))
    fq.fp8_quantize_block(xd, fmt, block_rows, qr, sr, qc, sc)
    return host(qr), host(sr), (host(qc) if colwise else None), (host(sc) if colwise else None)


def _check_block(x, fmt, block_rows):
    g = _gpu_block(x, fmt, block_rows)
    w = oracle.quantize_block(x, fmt, block_rows)
    for name, a, b in zip(("q_row", "s_row", "q_col", "s_col"), g, w):
        if a.dtype == np.float32:
            assert same_f32(a, b), name
        else:
            assert np.array_equal(a, b), (name, first_mismatches(a, b))


@pytest.mark.parametrize("block_rows", [128, 1])
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_block_small(block_rows, fmt, dt):
    rng = np.random.default_rng(block_rows)
    v = rng.standard_normal((384, 256)) * np.exp(rng.uniform(-8, 8, (384, 1)))
    v[:128, :128] = 0.0  # an all-zero block
    v[200, 3] = np.inf
    v[300, 130] = -np.inf
    v[140, 140] = np.nan
    x = v.astype(np.float32) if dt == "f32" else workloads.to_bf16_bits(v)
    _check_block(x, fmt, block_rows)


def test_block_weight_128x128_full_size():
    """7168x4096 bf16 weight, N(0, 0.02), 128x128 blocks, E4M3FN, with the
    transposed copy."""
    _check_block(workloads.block_weight(), E4, 128)


def test_block_activation_1x128_full_size():
    """4096x7168 bf16 activation with Student-t(3) channels, 1x128 blocks,
    E4M3FN, with the columnwise copy (128x1 blocks of x)."""
    _check_block(workloads.block_act(), E4, 1)


def test_block_rowwise_only():
    x = workloads.block_weight(256, 384, seed=3)
    g = _gpu_block(x, E5, 1, colwise=False)
    q_row, s_row = oracle.quantize_blocks(x, E5, 1, 128)
    assert np.array_equal(g[0], q_row) and same_f32(g[1], s_row)
