"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  Each one checks the oracle against something
other than itself: values the pages print, torch's float8 dtypes (a library
routine), numpy, brute force on small inputs, closed forms and invariants.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import read_golden

E4, E5 = oracle.E4M3FN, oracle.E5M2
TORCH_DT = {E4: torch.float8_e4m3fn, E5: torch.float8_e5m2}
MANT = {E4: 3, E5: 2}


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def torch_encode_clamped(y: np.ndarray, fmt: int) -> np.ndarray:
    """torch's float8 cast of values clamped to +-FP8_MAX first (torch's cast
    itself does not saturate).  NaN passes through the clamp."""
    fm = oracle.fmax(fmt)
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).clamp(-fm, fm)
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


# ----------------------------------------------------------- format pins ----
def test_format_constants_match_printed_values():
    """"Megatron FP8", section 2 prints (bias, e_max, max) = (7, 8, 448.0) and
    (15, 15, 57344.0) and the minimum normals 2^-6 / 2^-14."""
    for name, bias, emax, mx, lmin in read_golden("format_stats.txt"):
        fmt = E4 if name == "E4M3FN" else E5
        assert oracle.fmax(fmt) == float(mx)
        vals = oracle.decode_table(fmt)
        # bias: the exponent field of the code whose value is 1.0
        one = [c for c in range(128) if vals[c] == 1.0]
        assert len(one) == 1
        assert one[0] >> MANT[fmt] == int(bias)
        # e_max: exponent of the largest finite value
        assert math.floor(math.log2(oracle.fmax(fmt))) == int(emax)
        # min normal: the smallest code with a nonzero exponent field
        assert vals[1 << MANT[fmt]] == 2.0 ** int(lmin)
        assert all(0 < vals[c] < 2.0 ** int(lmin) for c in range(1, 1 << MANT[fmt]))


def test_decode_all_codes_matches_torch():
    """All 512 codes decode bit-identically to torch's float8 dtypes (NaN as a class)."""
    codes = torch.arange(256, dtype=torch.uint8)
    for fmt in (E4, E5):
        ref = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
        got = oracle.decode_table(fmt)
        nan = np.isnan(ref)
        assert np.array_equal(nan, np.isnan(got))
        assert np.array_equal(ref[~nan], got[~nan])
        assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_value_sets_counts_and_specials():
    """E4M3FN: 254 finite codes, 253 distinct values (+0 == -0), NaN only at
    0x7F/0xFF, no Inf.  E5M2: 248 finite codes, +-Inf at 0x7C/0xFC, six NaN codes."""
    v4, v5 = oracle.decode_table(E4), oracle.decode_table(E5)
    assert np.isfinite(v4).sum() == 254 and len(set(v4[np.isfinite(v4)])) == 253
    assert [c for c in range(256) if np.isnan(v4[c])] == [0x7F, 0xFF]
    assert not np.isinf(v4).any()
    assert np.isfinite(v5).sum() == 248 and len(set(v5[np.isfinite(v5)])) == 247
    assert v5[0x7C] == np.inf and v5[0xFC] == -np.inf
    assert [c for c in range(256) if np.isnan(v5[c])] == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    # non-negative finite codes are ordered by value
    for fmt, v in ((E4, v4), (E5, v5)):
        pos = v[: oracle.max_code(fmt) + 1]
        assert np.all(np.diff(pos) > 0)
        assert v[oracle.max_code(fmt)] == oracle.fmax(fmt)
        # E5M2 set equals the IEEE-style enumeration that skips the all-ones
        # exponent; E4M3FN adds the seven values 256..448 of that exponent
    assert len(v5[: 0x7C]) == 124
    assert sorted(v4[0x78:0x7F]) == [256.0, 288.0, 320.0, 352.0, 384.0, 416.0, 448.0]


# ----------------------------------------------------------- encode pins ----
def _probe_values(fmt: int) -> np.ndarray:
    """Inputs concentrated where encoders go wrong: every bf16 pattern at a few
    scales, every midpoint between neighbouring codes and its binary32
    neighbours, every code value and its neighbours, random bit patterns."""
    rng = np.random.default_rng(123 + fmt)
    all_bf16 = workloads.bf16_bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    with np.errstate(over="ignore", invalid="ignore"):
        parts = [all_bf16 * np.float32(s) for s in (1.0, 2.0 ** -7, 2.0 ** 7, 1.0 / 3.0, 3.7, 0.29877)]
    v = oracle.decode_table(fmt)[: oracle.max_code(fmt) + 1]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)  # midpoints are exact in binary32
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)
    pts = np.concatenate([mids, v.astype(np.float32), np.float32([oracle.fmax(fmt) * 1.0625])])
    b = pts.view(np.uint32).astype(np.int64)
    for d in (-2, -1, 1, 2):
        parts.append(np.clip(b + d, 0, 0x7F7FFFFF).astype(np.uint32).view(np.float32))
    parts.append(pts)
    parts.append(rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32))
    y = np.concatenate([p.astype(np.float32) for p in parts])
    return np.concatenate([y, -y])


@pytest.mark.parametrize("fmt", [E4, E5])
def test_encode_matches_torch_on_clamped_inputs(fmt):
    """torch's RNE float8 cast of pre-clamped values (a library routine) agrees
    with the oracle's nearest-value encode, NaN signs included."""
    y = _probe_values(fmt)
    got = oracle.encode(fmt, y)
    ref = torch_encode_clamped(y, fmt)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(int(f32_bits(y[i]))), hex(got[i]), hex(ref[i])) for i in bad[:10]]


@pytest.mark.parametrize("fmt", [E4, E5])
def test_encode_brute_force_nearest(fmt):
    """Exhaustive nearest search over all 256 decoded values (ties to the even
    code, sign copied) on random inputs: an independent statement of the
    definition."""
    rng = np.random.default_rng(7)
    fm = oracle.fmax(fmt)
    y = np.concatenate([rng.standard_normal(20000) * fm / 3, rng.standard_normal(20000) * fm * 1e-3,
                        rng.uniform(-2 * fm, 2 * fm, 5000)]).astype(np.float32)
    table = oracle.decode_table(fmt)
    finite = [c for c in range(256) if np.isfinite(table[c])]
    got = oracle.encode(fmt, y)
    for val, g in zip(y.astype(np.float64), got):
        a = min(abs(val), fm)
        best = None
        for c in finite:
            if (c >> 7) != int(np.signbit(val)):
                continue
            d = abs(abs(table[c]) - a)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                best = (d, c)
        assert g == best[1], (val, hex(g), hex(best[1]))


def test_encode_ties_golden():
    for row in read_golden("encode_ties.txt"):
        fmt = E4 if row[0] == "E4M3FN" else E5
        if len(row) == 5 and row[2] == "p":
            value = np.float32(float(row[1]) * 2.0 ** int(row[3]))
            code = int(row[4], 16)
        else:
            value = np.float32(float(row[1]))
            code = int(row[2], 16)
        assert oracle.encode(fmt, [value])[0] == code, (row, hex(oracle.encode(fmt, [value])[0]))


@pytest.mark.parametrize("fmt", [E4, E5])
def test_encode_invariants(fmt):
    table = oracle.decode_table(fmt)
    finite = [c for c in range(256) if np.isfinite(table[c])]
    # round trip of every finite code
    assert all(oracle.encode(fmt, [np.float32(table[c])])[0] == c for c in finite)
    # saturation and NaN
    fm = oracle.fmax(fmt)
    mc = oracle.max_code(fmt)
    sat = oracle.encode(fmt, np.float32([fm * 1.5, np.inf, -np.inf, -fm * 4, np.nan, -np.nan]))
    assert list(sat) == [mc, mc, 0x80 | mc, 0x80 | mc, 0x7F, 0xFF]
    # monotone in value
    rng = np.random.default_rng(1)
    y = np.sort(rng.uniform(-2 * fm, 2 * fm, 50000).astype(np.float32))
    dec = table[oracle.encode(fmt, y)]
    assert np.all(np.diff(dec) >= 0)
    # worst-case relative error 2^-(m+1) in the normal range ("Megatron FP8",
    # section 23); absolute error at most half the subnormal step below it
    m = MANT[fmt]
    min_normal = table[1 << m]
    yy = rng.uniform(0, fm, 200000).astype(np.float64)
    yy = np.concatenate([yy, rng.uniform(0, min_normal, 20000)]).astype(np.float32)
    dv = table[oracle.encode(fmt, yy)]
    yd = yy.astype(np.float64)
    normal = yd >= min_normal
    assert np.all(np.abs(dv[normal] - yd[normal]) <= yd[normal] * 2.0 ** -(m + 1))
    assert np.all(np.abs(dv[~normal] - yd[~normal]) <= table[1] / 2)


# ------------------------------------------------------ scaling pins --------
def test_amax_matches_numpy():
    x = workloads.tensor_fp32()
    assert oracle.amax(x) == np.abs(x).max() == np.float32(2000.0)
    xb = workloads.delayed_step(3, 256, 384)
    assert oracle.amax(xb) == np.abs(workloads.bf16_bits_to_f32(xb)).max()
    y = x.copy()
    y[5, 7] = -np.nan
    a = oracle.amax(y)
    assert np.isnan(a) and f32_bits(a) == 0x7FC00000
    assert oracle.amax(np.zeros(0, np.float32)) == 0.0
    assert oracle.amax(np.float32([-0.0, -3.0, np.inf])) == np.inf


def test_worked_example_scale():
    """"Megatron FP8", section 4: x = [-920, 3.5, 511], margin 1 gives
    s* = 920/448 and s = 2 s*."""
    g = {r[0]: r[1] for r in read_golden("worked_example.txt")}
    x = np.float32([g["x0"], g["x1"], g["x2"]])
    margin = int(g["margin"])
    a = oracle.amax(x)
    assert a == np.float32(g["amax"])
    s_star = np.float32(g["s_star_num"]) / np.float32(g["s_star_den"])
    s, sc = oracle.current_scale(a, E4, margin)
    assert s == s_star * np.float32(g["s_factor"])
    assert f32_bits(s) == 0x40836DB7
    assert sc == np.float32(1) / s and f32_bits(sc) == 0x3E79525D
    r = oracle.quantize_tensor(x, E4, amax_in=a, margin=margin)
    # codes of the scaled values by torch's cast (values already within +-448)
    ref = torch_encode_clamped(x * sc, E4)
    assert list(r["q"]) == list(ref) == [0xF6, 0x36, 0x70]
    # the amax element lands on FP8_MAX / 2^margin exactly
    assert oracle.decode(E4, r["q"][0]) == -448.0 / 2 ** margin
    assert list(oracle.dequantize(r["q"], E4, s)) == [np.float32(-224.0) * s, np.float32(0.875) * s,
                                                       np.float32(128.0) * s]


@pytest.mark.parametrize("fmt", [E4, E5])
def test_amax_element_lands_on_fmax(fmt):
    """Invariant: with current scaling and margin 0, an element equal to amax is
    encoded as +-FP8_MAX, whatever the amax (no overflow, no early clip)."""
    rng = np.random.default_rng(5)
    amaxes = np.exp(rng.uniform(np.log(1e-10), np.log(1e30), 20000)).astype(np.float32)
    mc = oracle.max_code(fmt)
    for a in amaxes:
        s, sc = oracle.current_scale(a, fmt, 0)
        q = oracle.quantize(np.float32([a, -a]), fmt, sc)
        assert list(q) == [mc, 0x80 | mc], (a, s, sc, q)


def test_current_scale_floor_and_specials():
    s, sc = oracle.current_scale(0.0, E4, 0)
    assert f32_bits(s) == 0x2720D7C5  # fl32(fl32(1e-12) / 448)
    s, sc = oracle.current_scale(np.float32(np.nan), E4, 0)
    assert np.isnan(s) and np.isnan(sc)
    s, sc = oracle.current_scale(np.float32(np.inf), E5, 0)
    assert s == np.inf and sc == 0.0
    # margin multiplies by an exact power of two
    s0, _ = oracle.current_scale(1234.5, E5, 0)
    for m in (-3, 1, 5):
        sm, _ = oracle.current_scale(1234.5, E5, m)
        assert sm == s0 * np.float32(2.0 ** m)


def test_tensor_fp32_scalars():
    x = workloads.tensor_fp32()
    r = oracle.quantize_tensor(x, E4, amax_in=oracle.amax(x), margin=1)
    assert r["amax"] == 2000.0
    assert f32_bits(r["scale_inv"]) == 0x410EDB6E and f32_bits(r["scale"]) == 0x3DE56041
    # the sixteen +-2000 outliers land on +-224 = 448 / 2^margin
    big = np.abs(x) == 2000.0
    assert big.sum() == 16
    assert set(r["q"][big].tolist()) <= {0x76, 0xF6}


def test_quantize_matches_torch_cast():
    """A whole tensor: oracle codes == torch cast of clamp(x * scale)."""
    for fmt in (E4, E5):
        x = workloads.tensor_fp32(256, 512, seed=11)
        s, sc = oracle.current_scale(oracle.amax(x), fmt, 1)
        assert np.array_equal(oracle.quantize(x, fmt, sc), torch_encode_clamped(x * sc, fmt))
        xb = workloads.delayed_step(2, 128, 256)
        s, sc = oracle.current_scale(oracle.amax(xb), fmt, 0)
        xf = workloads.bf16_bits_to_f32(xb)
        assert np.array_equal(oracle.quantize(xb, fmt, sc), torch_encode_clamped(xf * sc, fmt))


def test_dequantize_pins():
    codes = np.arange(256, dtype=np.uint8)
    for fmt in (E4, E5):
        ref = torch.from_numpy(codes).view(TORCH_DT[fmt]).float().numpy()
        for s in (1.0, 0.5, 2.0 ** 20):
            got = oracle.dequantize(codes, fmt, s)
            want = ref * np.float32(s)
            nan = np.isnan(want)
            assert np.array_equal(np.isnan(got), nan)
            assert np.array_equal(got[~nan], want[~nan])
    # quantize -> dequantize error bound (relative 2^-(m+1) above the normal
    # range of the scaled values)
    x = workloads.tensor_fp32(128, 128, seed=3)
    for fmt in (E4, E5):
        r = oracle.quantize_tensor(x, fmt, amax_in=oracle.amax(x), margin=0)
        y = oracle.dequantize(r["q"], fmt, r["scale_inv"]).astype(np.float64)
        xs = np.abs(x.astype(np.float64))
        min_normal = oracle.decode(fmt, 1 << MANT[fmt]) * float(r["scale_inv"])
        n = xs >= min_normal
        assert np.all(np.abs(y[n] - x[n]) <= xs[n] * 2.0 ** -(MANT[fmt] + 1) * (1 + 1e-6))


def test_rowwise_colwise_is_transpose():
    x = workloads.delayed_step(1, 192, 320)
    s, sc = oracle.current_scale(oracle.amax(x), E5, 0)
    q_row, q_col = oracle.quantize_rowwise_colwise(x, E5, sc)
    assert np.array_equal(q_row, oracle.quantize(x, E5, sc))
    assert np.array_equal(q_col, q_row.T)
    assert np.array_equal(oracle.transpose(x), x.T)


# ---------------------------------------------------------- delayed pins ----
def test_delayed_ring_golden():
    rows = read_golden("delayed_ring.txt")
    hist = np.zeros((2, 1), np.float32)
    scale = np.ones(1, np.float32)
    scale_inv = np.ones(1, np.float32)
    for step, a, s_used, ring in rows:
        assert scale_inv[0] == np.float32(s_used), (step, scale_inv)
        assert scale[0] == np.float32(1) / np.float32(s_used)
        oracle.delayed_update(hist, 0, np.float32(a), int(step), E4, 0, oracle.ALGO_MAX, scale, scale_inv)
        assert list(hist[:, 0]) == [float(v) for v in ring.split(",")]


def test_delayed_replay_invariants():
    """32 updates on one shared ring of 16 with alternating formats: the ring
    holds the last 16 amaxes at slot t % 16 and each scale is max(window) /
    FP8_MAX of the format that consumes it; "most_recent" uses only the value
    just written; a second column is untouched by updates of the first."""
    rng = np.random.default_rng(9)
    amaxes = np.float32(np.abs(rng.standard_normal(32)) * 3)
    hist = np.zeros((16, 2), np.float32)
    hist[:, 1] = 7.0
    scale = np.ones(2, np.float32)
    scale_inv = np.ones(2, np.float32)
    for t in range(32):
        fmt_next = E4 if (t + 1) % 2 == 0 else E5
        oracle.delayed_update(hist, 0, amaxes[t], t, fmt_next, 0, oracle.ALGO_MAX, scale, scale_inv)
        window = amaxes[max(0, t - 15): t + 1]
        assert scale_inv[0] == window.max() / np.float32(oracle.fmax(fmt_next))
        assert hist[t % 16, 0] == amaxes[t]
    assert np.array_equal(hist[:, 0], amaxes[16:])
    assert np.all(hist[:, 1] == 7.0) and scale[1] == 1.0
    h2 = np.zeros((4, 1), np.float32)
    sc2, si2 = np.ones(1, np.float32), np.ones(1, np.float32)
    for t, a in enumerate([5.0, 1.0, 3.0]):
        oracle.delayed_update(h2, 0, a, t, E4, 2, oracle.ALGO_MOST_RECENT, sc2, si2)
        assert si2[0] == np.float32(a) / np.float32(448) * np.float32(4)
    # a NaN in the window: eff is NaN, not > 0, so the factor falls back to 1
    oracle.delayed_update(h2, 0, np.float32(np.nan), 3, E4, 0, oracle.ALGO_MAX, sc2, si2)
    assert si2[0] == 1.0 and sc2[0] == 1.0


# ------------------------------------------------------------ block pins ----
def test_block_128x128_invariants():
    x = workloads.block_weight(384, 256, seed=21)
    x[:128, :128] = 0  # an all-zero block
    q_row, s_row, q_col, s_col = oracle.quantize_block(x, E4, 128)
    assert q_row.shape == (384, 256) and s_row.shape == (3, 2)
    assert np.array_equal(q_col, q_row.T) and np.array_equal(s_col, s_row.T)
    assert f32_bits(s_row[0, 0]) == 0x2720D7C5 and np.all(q_row[:128, :128] == 0)
    for I in range(3):
        for J in range(2):
            blk = np.ascontiguousarray(x[I * 128:(I + 1) * 128, J * 128:(J + 1) * 128])
            # a block is quantized exactly like a tensor of its own with current scaling
            r = oracle.quantize_tensor(blk, E4, amax_in=oracle.amax(blk), margin=0)
            assert s_row[I, J] == r["scale_inv"]
            assert np.array_equal(q_row[I * 128:(I + 1) * 128, J * 128:(J + 1) * 128], r["q"])
            if (I, J) != (0, 0):
                assert np.any((q_row[I * 128:(I + 1) * 128, J * 128:(J + 1) * 128] & 0x7F) == 0x7E)


def test_block_1x128_invariants():
    x = workloads.block_act(256, 384, seed=22)
    q_row, s_row, q_col, s_col = oracle.quantize_block(x, E4, 1)
    assert s_row.shape == (256, 3) and q_col.shape == (384, 256) and s_col.shape == (384, 2)
    xf = workloads.bf16_bits_to_f32(x)
    for i in (0, 17, 255):
        for J in range(3):
            seg = np.ascontiguousarray(x[i, J * 128:(J + 1) * 128])
            r = oracle.quantize_tensor(seg, E4, amax_in=oracle.amax(seg))
            assert s_row[i, J] == r["scale_inv"]
            assert np.array_equal(q_row[i, J * 128:(J + 1) * 128], r["q"])
    for j in (0, 200, 383):
        for I in range(2):
            seg = np.ascontiguousarray(x[I * 128:(I + 1) * 128, j])
            r = oracle.quantize_tensor(seg, E4, amax_in=oracle.amax(seg))
            assert s_col[j, I] == r["scale_inv"]
            assert np.array_equal(q_col[j, I * 128:(I + 1) * 128], r["q"])
    # every row segment contains its +-FP8_MAX
    assert np.all(np.any((q_row.reshape(256, 3, 128) & 0x7F) == 0x7E, axis=2) | (
        np.abs(xf).reshape(256, 3, 128).max(axis=2) == 0))


# ------------------------------------------------------------- GEMM pins ----
def _brute_gemm(A, fa, sA, B, fb, sB, mode):
    ta, tb = oracle.decode_table(fa), oracle.decode_table(fb)
    M, K = A.shape
    N = B.shape[0]
    R = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                w = ta[A[m, k]] * tb[B[n, k]]
                if mode == oracle.PER_TENSOR:
                    acc += w
                elif mode == oracle.BLOCK_1x128_128x128:
                    acc += w * sA[m, k // 128] * sB[n // 128, k // 128]
                else:
                    acc += w * sA[m, k // 128] * sB[n, k // 128]
            R[m, n] = acc * (float(sA) * float(sB) if mode == oracle.PER_TENSOR else 1.0)
    return R


def _random_codes(rng, shape, fmt):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    t = oracle.decode_table(fmt)
    bad = ~np.isfinite(t[c])
    c[bad] = 0x38
    return c


def test_gemm_reference_brute_force_per_tensor():
    rng = np.random.default_rng(31)
    A = _random_codes(rng, (5, 256), E4)
    B = _random_codes(rng, (7, 256), E5)
    R = oracle.gemm_reference(A, E4, np.float32(0.75), B, E5, np.float32(3.0))
    assert np.allclose(R, _brute_gemm(A, E4, np.float32(0.75), B, E5, np.float32(3.0), oracle.PER_TENSOR),
                       rtol=1e-12, atol=0)
    ent = oracle.gemm_reference_entries(A, E4, np.float32(0.75), B, E5, np.float32(3.0), [0, 4, 2], [6, 0, 3])
    assert np.allclose(ent, R[[0, 4, 2], [6, 0, 3]], rtol=1e-12, atol=0)


def test_gemm_reference_brute_force_block():
    rng = np.random.default_rng(32)
    M, N, K = 3, 256, 384
    A = _random_codes(rng, (M, K), E5)
    B = _random_codes(rng, (N, K), E4)
    sA = np.float32(rng.uniform(0.1, 2, (M, K // 128)))
    sB = np.float32(rng.uniform(0.1, 2, (N // 128, K // 128)))
    R = oracle.gemm_reference(A, E5, sA, B, E4, sB, oracle.BLOCK_1x128_128x128)
    ref = _brute_gemm(A, E5, sA, B, E4, sB, oracle.BLOCK_1x128_128x128)
    assert np.allclose(R, ref, rtol=1e-12, atol=1e-300)
    ent = oracle.gemm_reference_entries(A, E5, sA, B, E4, sB, [2, 0], [255, 129], oracle.BLOCK_1x128_128x128)
    assert np.allclose(ent, ref[[2, 0], [255, 129]], rtol=1e-12, atol=0)


def test_gemm_reference_brute_force_block_1x128_both():
    """The weight-gradient layout: both operands carry 1x128 scales, B's per row."""
    rng = np.random.default_rng(34)
    M, N, K = 4, 6, 384
    A = _random_codes(rng, (M, K), E5)
    B = _random_codes(rng, (N, K), E4)
    sA = np.float32(rng.uniform(0.1, 2, (M, K // 128)))
    sB = np.float32(rng.uniform(0.1, 2, (N, K // 128)))
    R = oracle.gemm_reference(A, E5, sA, B, E4, sB, oracle.BLOCK_1x128_1x128)
    ref = _brute_gemm(A, E5, sA, B, E4, sB, oracle.BLOCK_1x128_1x128)
    assert np.allclose(R, ref, rtol=1e-12, atol=1e-300)
    ent = oracle.gemm_reference_entries(A, E5, sA, B, E4, sB, [3, 0], [5, 1], oracle.BLOCK_1x128_1x128)
    assert np.allclose(ent, ref[[3, 0], [5, 1]], rtol=1e-12, atol=0)
    # B's 1x128 scales that are equal within each 128-row group reduce to the 128x128 rule
    N2 = 256
    B2 = _random_codes(rng, (N2, K), E4)
    sB_blk = np.float32(rng.uniform(0.1, 2, (N2 // 128, K // 128)))
    sB_rows = np.repeat(sB_blk, 128, axis=0)
    assert np.array_equal(oracle.gemm_reference(A, E5, sA, B2, E4, sB_rows, oracle.BLOCK_1x128_1x128),
                          oracle.gemm_reference(A, E5, sA, B2, E4, sB_blk, oracle.BLOCK_1x128_128x128))


def test_gemm_abs_sum_bounds_the_result():
    """S >= |R| everywhere, S == R when every term is non-negative, and S is the
    brute-force sum of absolute terms."""
    rng = np.random.default_rng(35)
    M, N, K = 3, 5, 256
    A = _random_codes(rng, (M, K), E4)
    B = _random_codes(rng, (N, K), E5)
    sA = np.float32(rng.uniform(-2, 2, (M, K // 128)))
    sB = np.float32(rng.uniform(-2, 2, (N, K // 128)))
    for mode, a_s, b_s in ((oracle.PER_TENSOR, np.float32(-0.5), np.float32(3.0)),
                           (oracle.BLOCK_1x128_1x128, sA, sB)):
        R = oracle.gemm_reference(A, E4, a_s, B, E5, b_s, mode)
        S = oracle.gemm_abs_sum(A, E4, a_s, B, E5, b_s, mode)
        assert np.all(S >= np.abs(R) * (1 - 1e-12))
        ta, tb = np.abs(oracle.decode_table(E4)), np.abs(oracle.decode_table(E5))
        m, n = 2, 4
        terms = ta[A[m]] * tb[B[n]]
        if mode == oracle.PER_TENSOR:
            brute = terms.sum() * abs(float(a_s) * float(b_s))
        else:
            brute = sum(terms[kb * 128:(kb + 1) * 128].sum() * abs(float(a_s[m, kb]) * float(b_s[n, kb]))
                        for kb in range(K // 128))
        assert np.isclose(S[m, n], brute, rtol=1e-12)
    Ap = A & 0x7F
    Bp = B & 0x7F
    Rp = oracle.gemm_reference(Ap, E4, np.abs(sA), Bp, E5, np.abs(sB), oracle.BLOCK_1x128_1x128)
    Sp = oracle.gemm_abs_sum(Ap, E4, np.abs(sA), Bp, E5, np.abs(sB), oracle.BLOCK_1x128_1x128)
    assert np.allclose(Rp, Sp, rtol=1e-12)


def test_gemm_reference_exact_special_cases():
    """Entries in {0, +-1}: integer sums; all-ones block scales reduce block
    mode to the per-tensor product; A = 0 gives 0."""
    rng = np.random.default_rng(33)
    one, m_one, zero = 0x38, 0xB8, 0x00
    A = rng.choice(np.uint8([one, m_one, zero]), (16, 128))
    B = rng.choice(np.uint8([one, m_one, zero]), (24, 128))
    av = np.where(A == one, 1, np.where(A == m_one, -1, 0))
    bv = np.where(B == one, 1, np.where(B == m_one, -1, 0))
    R = oracle.gemm_reference(A, E4, 1.0, B, E4, 1.0)
    assert np.array_equal(R, (av @ bv.T).astype(np.float64))
    Rb = oracle.gemm_reference(A, E4, np.ones((16, 1), np.float32), B, E4, np.ones((1, 1), np.float32),
                               oracle.BLOCK_1x128_128x128)
    assert np.array_equal(Rb, R)
    assert not oracle.gemm_reference(np.zeros_like(A), E4, 1.0, B, E4, 1.0).any()


def test_nan_product_sign_rule():
    """NaN products take sign(x) XOR sign(scale) (the sign rule of
    multiplication; IEEE 754 leaves an invalid product's NaN sign open)."""
    nan = np.float32(np.nan)
    x = np.float32([np.inf, -np.inf, 1.0, -nan, nan, -2.0])
    assert list(oracle.quantize(x, E4, np.float32(0.0))) == [0x7F, 0xFF, 0x00, 0xFF, 0x7F, 0x80]
    assert list(oracle.quantize(x, E5, nan)) == [0x7F, 0xFF, 0x7F, 0xFF, 0x7F, 0xFF]
    assert list(oracle.quantize(x, E4, np.float32(-1.0))) == [0xFE, 0x7E, 0xB8, 0x7F, 0xFF, 0x40]


# ---------------------------------------------------------------- MXFP8 pins --
def test_e8m0_scale_values():
    """E8M0 ("Megatron FP8", sections 10 and 16): an unsigned exponent byte, no
    mantissa, no sign; powers of two from 2^-127 to 2^127; 255 is NaN."""
    v = oracle.e8m0_value(np.arange(256))
    assert v[0] == 2.0 ** -127 and v[127] == 1.0 and v[254] == 2.0 ** 127
    assert np.isnan(v[255])
    assert np.all(v[1:255] == 2 * v[0:254])


def test_mx_scale_overhead_page_example():
    """Section 16's count: 1,048,576 FP8 elements carry 32,768 scale bytes
    (one per 32), 1,081,344 bytes in all (3.125% metadata)."""
    x = np.float32(np.random.default_rng(40).standard_normal((1024, 1024)))
    q, sc = oracle.quantize_mx(x, E4)
    assert q.size == 1048576 and sc.size == 32768 and q.nbytes + sc.nbytes == 1081344


@pytest.mark.parametrize("fmt,emax,mbits", [(E4, 8, 3), (E5, 15, 2)])
def test_mx_block_max_in_top_binade_and_error_bound(fmt, emax, mbits):
    """Every block's largest element lands in the format's top binade
    [2^emax, 2^(emax+1)) after scaling (so the block uses the format's whole
    range), and every element reconstructs within half a unit in the last place
    of its binade (2^-(m+1) relative, section 24's bound), or saturates at
    FP8_MAX, which only the top binade's values above FP8_MAX do."""
    rng = np.random.default_rng(41 + fmt)
    x64 = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    x = np.float32(x64)
    q, sc = oracle.quantize_mx(x, fmt)
    tab = oracle.decode_table(fmt)
    fmax = oracle.fmax(fmt)
    e = sc.astype(np.int64) - 127
    xs = x.astype(np.float64) * np.ldexp(1.0, -np.repeat(e, 32, axis=1))  # exact scaled values
    blk_max = np.abs(xs).reshape(64, 8, 32).max(axis=2)
    assert np.all((blk_max >= 2.0 ** emax) & (blk_max < 2.0 ** (emax + 1)))
    dec = tab[q]
    sat = np.abs(xs) > fmax
    assert np.all(np.abs(dec[sat]) == fmax)
    normal = (~sat) & (np.abs(xs) >= 2.0 ** (1 - (7 if fmt == E4 else 15)))
    binade = np.ldexp(1.0, np.floor(np.log2(np.abs(xs[normal]))).astype(int))
    assert np.all(np.abs(dec[normal] - xs[normal]) <= binade * 2.0 ** -(mbits + 1))
    sub = (~sat) & ~normal
    step = 2.0 ** ((1 - (7 if fmt == E4 else 15)) - mbits)
    assert np.all(np.abs(dec[sub] - xs[sub]) <= step / 2)


def test_mx_special_blocks():
    """All-zero block: scale 2^-127 (byte 0), codes 0.  A block of one power of
    two 2^k: scale 2^(k - emax), every code the format's 2^emax (0x78 in both
    formats).  A NaN in the block: NaN scale byte and NaN codes."""
    x = np.zeros((3, 64), np.float32)
    x[1, :32] = 2.0 ** 5
    x[1, 32:] = -(2.0 ** -30)
    x[2, :32] = np.float32(1.5)
    x[2, 7] = np.nan
    for fmt, emax in ((E4, 8), (E5, 15)):
        q, sc = oracle.quantize_mx(x, fmt)
        assert list(sc[0]) == [0, 0] and not q[0].any()
        assert sc[1, 0] == 5 - emax + 127 and np.all(q[1, :32] == 0x78)
        assert sc[1, 1] == -30 - emax + 127 and np.all(q[1, 32:] == 0xF8)
        assert sc[2, 0] == 255 and np.all((q[2, :32] & 0x7F) == 0x7F)


def test_mx_colwise_is_rowwise_of_transpose():
    x = np.float32(np.random.default_rng(42).standard_normal((64, 96)))
    qc, sc = oracle.quantize_mx_colwise(x, E5)
    qt, st = oracle.quantize_mx(np.ascontiguousarray(x.T), E5)
    assert np.array_equal(qc, qt) and np.array_equal(sc, st) and qc.shape == (96, 64)


def test_gemm_reference_mx():
    """MXFP8 GEMM: unit scales (byte 127) reduce to the unscaled product;
    brute force on a tiny case; a power-of-two scale on one block of A scales
    exactly that block's contribution."""
    rng = np.random.default_rng(43)
    M, N, K = 3, 4, 96
    A = _random_codes(rng, (M, K), E4)
    B = _random_codes(rng, (N, K), E5)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    R1 = oracle.gemm_reference(A, E4, ones_a, B, E5, ones_b, oracle.MXFP8)
    assert np.array_equal(R1, oracle.gemm_reference(A, E4, 1.0, B, E5, 1.0))
    sa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    R = oracle.gemm_reference(A, E4, sa, B, E5, sb, oracle.MXFP8)
    ta, tb = oracle.decode_table(E4), oracle.decode_table(E5)
    for m in range(M):
        for n in range(N):
            ref = sum(ta[A[m, k]] * 2.0 ** (int(sa[m, k // 32]) - 127) * tb[B[n, k]] * 2.0 ** (int(sb[n, k // 32]) - 127)
                      for k in range(K))
            assert np.isclose(R[m, n], ref, rtol=1e-12, atol=0)
    ent = oracle.gemm_reference_entries(A, E4, sa, B, E5, sb, [2, 0], [3, 1], oracle.MXFP8)
    assert np.allclose(ent, R[[2, 0], [3, 1]], rtol=1e-12, atol=0)
    sa2 = sa.copy()
    sa2[1, 2] += 3
    R2 = oracle.gemm_reference(A, E4, sa2, B, E5, sb, oracle.MXFP8)
    part = oracle.gemm_reference(A[:, 64:96], E4, sa[:, 2:3], B[:, 64:96], E5, sb[:, 2:3], oracle.MXFP8)
    assert np.allclose(R2[1] - R[1], 7 * part[1], rtol=1e-12, atol=1e-300)
    assert np.array_equal(R2[[0, 2]], R[[0, 2]])


# ---------------------------------------------------------- GEMM epilogue ----
# Standard normal CDF values as printed in statistical tables (and the erf(1)
# constant); GELU(x) = x * Phi(x).
PHI_TABLE = [(0.0, 0.5), (1.0, 0.8413447460685429), (-1.0, 0.15865525393145707), (2.0, 0.9772498680518208),
             (3.0, 0.9986501019683699), (-3.0, 0.0013498980316301035), (1.959963984540054, 0.975)]
ERF_1 = 0.8427007929497149


def test_gelu_tabulated_values():
    """A wrong sign inside Phi gives GELU(1) = 0.159, a missing 1/sqrt 2 gives
    0.921; both fail here."""
    for x, phi in PHI_TABLE:
        assert math.isclose(float(oracle.gelu(x)), x * phi, rel_tol=1e-12, abs_tol=1e-300), x


def test_gelu_invariants_and_tails():
    x = np.linspace(-8, 8, 4001)
    g = oracle.gelu(x)
    # x Phi(x) - (-x) Phi(-x) = x (Phi(x) + Phi(-x)) = x
    assert np.allclose(g - oracle.gelu(-x), x, rtol=0, atol=1e-14)
    # the minimum is about -0.17, near x = -0.75
    i = int(np.argmin(g))
    assert -0.1701 < g[i] < -0.1699 and -0.76 < x[i] < -0.74
    assert oracle.gelu(40.0) == 40.0 and oracle.gelu(0.0) == 0.0
    # far left tail: x Phi(x) ~ phi(x) (1 - 1/x^2 + ...) (Mills ratio)
    t = -10.0
    mills = math.exp(-t * t / 2) / math.sqrt(2 * math.pi) * (1 - 1 / t ** 2 + 3 / t ** 4 - 15 / t ** 6)
    assert math.isclose(float(oracle.gelu(t)), -mills, rel_tol=1e-4)
    assert np.isnan(oracle.gelu(np.nan)) and np.isnan(oracle.gelu(-np.inf))
    assert oracle.gelu(np.inf) == np.inf


def test_gelu_slope_bound():
    """The slope Phi(x) + x phi(x) peaks at x = sqrt 2 at
    Phi(sqrt 2) + sqrt 2 phi(sqrt 2) = (1 + erf 1)/2 + e^-1 / sqrt(pi) ~ 1.1289
    and bottoms at -0.1289 (x = -sqrt 2): the factor by which GELU can grow an
    error of its argument (the GPU tests use 1.13)."""
    peak = (1 + ERF_1) / 2 + math.exp(-1) / math.sqrt(math.pi)
    x = np.linspace(-10, 10, 400001)
    d = np.diff(oracle.gelu(x)) / np.diff(x)
    assert abs(d.max() - peak) < 1e-6 and abs(d.min() - (1 - peak)) < 1e-6
    assert peak < 1.13


def test_relu_and_epilogue_composition():
    v = np.array([-1.0, -0.0, 0.0, 2.5, np.nan])
    r = oracle.relu(v)
    assert r[0] == 0 and not np.signbit(r[0]) and np.signbit(r[1]) and r[3] == 2.5 and np.isnan(r[4])
    # bias is per output column: R [2][3] + bias [3]
    R = np.array([[1.0, -2.0, 3.0], [-4.0, 5.0, -6.0]])
    b = np.array([0.5, 1.0, 10.0])
    assert np.array_equal(oracle.epilogue_reference(R, b), [[1.5, -1.0, 13.0], [-3.5, 6.0, 4.0]])
    assert np.array_equal(oracle.epilogue_reference(R, b, oracle.ACT_RELU), [[1.5, 0.0, 13.0], [0.0, 6.0, 4.0]])
    with pytest.raises(ValueError):
        oracle.epilogue_reference(R, np.ones(2))
    # the activation applies after the bias
    g = oracle.epilogue_reference(np.array([[-1.0]]), np.array([2.0]), oracle.ACT_GELU)
    assert math.isclose(float(g[0, 0]), 0.8413447460685429, rel_tol=1e-12)


def test_epilogue_gemm_brute_force():
    """GEMM + bias + GELU on a tiny case by loops over the decode table."""
    rng = np.random.default_rng(71)
    M, N, K = 3, 5, 128
    A = rng.integers(0, 0x7F, (M, K)).astype(np.uint8)
    B = rng.integers(0, 0x7B, (N, K)).astype(np.uint8) | 0x80 * rng.integers(0, 2, (N, K)).astype(np.uint8)
    sA, sB = np.float32(0.37), np.float32(0.011)
    bias = rng.standard_normal(N)
    y = oracle.epilogue_reference(oracle.gemm_reference(A, E4, sA, B, E5, sB), bias, oracle.ACT_GELU)
    for m in range(M):
        for n in range(N):
            acc = sum(oracle.decode(E4, int(A[m, k])) * oracle.decode(E5, int(B[n, k])) for k in range(K))
            v = acc * float(sA) * float(sB) + bias[n]
            want = v * 0.5 * (1 + math.erf(v / math.sqrt(2)))
            assert math.isclose(y[m, n], want, rel_tol=1e-12, abs_tol=1e-15)


def test_epilogue_fp8_output_codes():
    """FP8 output with dequant scale s = 2: the values are multiplied by
    fl32(1/2) = 0.5 and cast: 1 -> 0.5 (0x30), 896 -> 448 (0x7E), -3 -> -1.5
    (0xBC), 2000 -> 1000 saturates to 448; the amax is taken before the cast."""
    q, am = oracle.epilogue_fp8_codes(np.array([[1.0, 896.0, -3.0, 2000.0]]), E4, 2.0)
    assert q.tolist() == [[0x30, 0x7E, 0xBC, 0x7E]] and am == 2000.0
    # E5M2: 57344 is the largest finite value, and 1000 * 0.5 = 500 lies
    # between 448 and 512 (step 64 in [256, 512)): 512 is nearer
    q, am = oracle.epilogue_fp8_codes(np.array([[1000.0, -0.25]]), E5, 2.0)
    assert [oracle.decode(E5, int(c)) for c in q[0]] == [512.0, -0.125]


# ------------------------------------ per-direction quantization, diagnostics ----
def test_hybrid_same_format_is_rowwise_colwise():
    """One format, one scale, columnwise from the original: the hybrid
    quantizer reduces to the rowwise + columnwise cast (pinned above)."""
    x = workloads.delayed_step(3, 256, 384)
    am = oracle.amax(x)
    for fmt in (E4, E5):
        h = oracle.quantize_hybrid(x, fmt, fmt, oracle.COLSRC_ORIGINAL, amax_in=am, row_margin=1, col_margin=1)
        s, sc = oracle.current_scale(am, fmt, 1)
        q_row, q_col = oracle.quantize_rowwise_colwise(x, fmt, sc)
        assert np.array_equal(h["q_row"], q_row) and np.array_equal(h["q_col"], q_col)
        assert f32_bits(h["row_scale_inv"]) == f32_bits(s) == f32_bits(h["col_scale_inv"])


def test_hybrid_cross_format_directions_are_independent():
    """E4M3 rows and E5M2 columns from the original: each copy is the
    per-tensor cast of x (resp. x^T) in its own format, with its own margin."""
    x = workloads.block_act(128, 256, seed=4)
    am = oracle.amax(x)
    h = oracle.quantize_hybrid(x, E4, E5, oracle.COLSRC_ORIGINAL, amax_in=am, row_margin=0, col_margin=2)
    r = oracle.quantize_tensor(x, E4, amax_in=am, margin=0)
    c = oracle.quantize_tensor(oracle.transpose(x), E5, amax_in=am, margin=2)
    assert np.array_equal(h["q_row"], r["q"]) and np.array_equal(h["q_col"], c["q"])


SUBQ = (oracle.SUBQ_BLOCK_128x128, oracle.SUBQ_BLOCK_1x128, oracle.SUBQ_MXFP8)
TOP_CODE = {E4: 0x7E, E5: 0x7B}  # +FP8_MAX: 448 = 1.75 * 2^8, 57344 = 1.75 * 2^15


@pytest.mark.parametrize("recipe", SUBQ)
def test_hybrid_blockwise_one_format_is_the_single_recipe(recipe):
    """One format in both directions: the per-direction quantizer with block
    sub-quantizers reduces to the block (resp. MXFP8) quantizer with its
    columnwise copy, both pinned above."""
    x = workloads.block_act(256, 384, seed=23)
    for fmt in (E4, E5):
        h = oracle.quantize_hybrid_blockwise(x, recipe, fmt, recipe, fmt)
        if recipe == oracle.SUBQ_MXFP8:
            want = oracle.quantize_mx(x, fmt) + oracle.quantize_mx_colwise(x, fmt)
        else:
            want = oracle.quantize_block(x, fmt, 128 if recipe == oracle.SUBQ_BLOCK_128x128 else 1)
        for got, w in zip((h["q_row"], h["s_row"], h["q_col"], h["s_col"]), want):
            assert got.dtype == w.dtype and np.array_equal(got, w)


def test_hybrid_blockwise_cross_format_blocks_are_independent_tensors():
    """E4M3 rows and E5M2 columns, 128x128 blocks: every block of the
    columnwise copy is the per-tensor current-scaling cast of that block of
    x^T in E5M2 (torch-pinned above), every block of the rowwise copy that of
    x in E4M3; a block's maximum takes its own format's top code."""
    x = workloads.block_weight(256, 384, seed=24, std=3.0)
    h = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_BLOCK_128x128, E4, oracle.SUBQ_BLOCK_128x128, E5)
    assert h["s_row"].shape == (2, 3) and h["s_col"].shape == (3, 2) and h["q_col"].shape == (384, 256)
    for I in range(2):
        for J in range(3):
            rs, cs = slice(I * 128, (I + 1) * 128), slice(J * 128, (J + 1) * 128)
            blk = np.ascontiguousarray(x[rs, cs])
            r = oracle.quantize_tensor(blk, E4, amax_in=oracle.amax(blk))
            c = oracle.quantize_tensor(np.ascontiguousarray(blk.T), E5, amax_in=oracle.amax(blk))
            assert h["s_row"][I, J] == r["scale_inv"] and np.array_equal(h["q_row"][rs, cs], r["q"])
            assert h["s_col"][J, I] == c["scale_inv"] and np.array_equal(h["q_col"][cs, rs], c["q"])
            assert np.any((h["q_row"][rs, cs] & 0x7F) == TOP_CODE[E4])
            assert np.any((h["q_col"][cs, rs] & 0x7F) == TOP_CODE[E5])


def test_hybrid_blockwise_cross_recipe_directions():
    """MXFP8 E4M3 rows with 1x128 E5M2 columns: the rowwise copy is MXFP8 of
    x; each 128-row segment of a column is a tensor of its own cast to E5M2,
    whose maximum takes E5M2's top code."""
    x = workloads.block_act(256, 256, seed=25)
    h = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_MXFP8, E4, oracle.SUBQ_BLOCK_1x128, E5)
    q, sc = oracle.quantize_mx(x, E4)
    assert np.array_equal(h["q_row"], q) and np.array_equal(h["s_row"], sc)
    assert h["q_col"].shape == (256, 256) and h["s_col"].shape == (256, 2) and h["s_col"].dtype == np.float32
    xf = workloads.bf16_bits_to_f32(x)
    for j in (0, 77, 255):
        for I in range(2):
            seg = np.ascontiguousarray(x[I * 128:(I + 1) * 128, j])
            r = oracle.quantize_tensor(seg, E5, amax_in=oracle.amax(seg))
            assert h["s_col"][j, I] == r["scale_inv"]
            assert np.array_equal(h["q_col"][j, I * 128:(I + 1) * 128], r["q"])
            if np.abs(xf[I * 128:(I + 1) * 128, j]).max() > 0:
                assert np.any((h["q_col"][j, I * 128:(I + 1) * 128] & 0x7F) == TOP_CODE[E5])


def test_hybrid_blockwise_dequantized_128x128_one_format_is_the_transpose():
    """128x128 blocks, one format, columns from the dequantized rows: a block
    requantized from its own dequantized values gives back its codes (the FP8
    grid is far coarser than the binary32 roundings of x' and of the new
    scale), so q_col is q_row^T and s_col is s_row^T to within one binary32
    step.  A block holding a NaN keeps its NaN codes; a block holding +inf
    has scale inf, zero codes for its finite elements and x' = 0 * inf = NaN
    everywhere, so every column code is the NaN code with the row code's sign."""
    x = workloads.block_weight(384, 256, seed=26, std=3.0)
    x[5, 9] = 0x7FC0         # NaN in block (0, 0)
    x[130, 140] = 0x7F80     # +inf in block (1, 1)
    x[131, 141] = 0xC000     # -2.0 in the same block
    h = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_BLOCK_128x128, E4, oracle.SUBQ_BLOCK_128x128, E4,
                                         oracle.COLSRC_ROWWISE_DEQUANTIZED)
    qr, qc = h["q_row"], h["q_col"]
    for I in range(3):
        for J in range(2):
            rs, cs = slice(I * 128, (I + 1) * 128), slice(J * 128, (J + 1) * 128)
            if (I, J) == (1, 1):
                assert np.isinf(h["s_row"][I, J]) and np.isnan(h["s_col"][J, I])
                assert qr[131, 141] == 0x80 and (qr[130, 140] & 0x7F) == 0x7F
                assert np.array_equal(qc[cs, rs], (qr[rs, cs] | 0x7F).T)
            elif (I, J) == (0, 0):
                assert np.isnan(h["s_row"][I, J]) and np.all((qr[rs, cs] & 0x7F) == 0x7F)
                assert np.array_equal(qc[cs, rs], qr[rs, cs].T)
            else:
                assert np.array_equal(qc[cs, rs], qr[rs, cs].T)
                d = int(f32_bits(h["s_col"][J, I])) - int(f32_bits(h["s_row"][I, J]))
                assert abs(d) <= 1


def test_hybrid_blockwise_dequantized_mx_rows_exact_values():
    """MXFP8 E4M3 rows, 1x128 E5M2 columns from the dequantized rows: x' is
    the E4M3 value times the row block's power of two (computed here in
    float64, exact), and each 128-row segment of a column of x' is a tensor
    of its own cast to E5M2 (pinned above)."""
    x = workloads.block_act(256, 256, seed=27)
    h = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_MXFP8, E4, oracle.SUBQ_BLOCK_1x128, E5,
                                         oracle.COLSRC_ROWWISE_DEQUANTIZED)
    q, sc = oracle.quantize_mx(x, E4)
    assert np.array_equal(h["q_row"], q) and np.array_equal(h["s_row"], sc)
    xp = oracle.decode_table(E4)[q] * np.ldexp(1.0, np.repeat(sc.astype(np.int64) - 127, 32, axis=1))
    xp32 = xp.astype(np.float32)
    assert np.array_equal(xp32.astype(np.float64), xp)  # every x' fits binary32
    for j in (0, 31, 128, 255):
        for I in range(2):
            seg = np.ascontiguousarray(xp32[I * 128:(I + 1) * 128, j])
            r = oracle.quantize_tensor(seg, E5, amax_in=oracle.amax(seg))
            assert h["s_col"][j, I] == r["scale_inv"]
            assert np.array_equal(h["q_col"][j, I * 128:(I + 1) * 128], r["q"])
    # the original source gives other codes somewhere (the rows' rounding moved x)
    o = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_MXFP8, E4, oracle.SUBQ_BLOCK_1x128, E5)
    assert not np.array_equal(o["q_col"], h["q_col"])


def test_hybrid_blockwise_with_one_per_tensor_direction():
    """A per-tensor direction paired with a block one: per-tensor E4M3 rows
    (current scaling, margin 1) with MXFP8 E5M2 columns reduce to the
    per-tensor cast and the columnwise MXFP8 copy (both pinned above); 1x128
    rows with per-tensor E5M2 columns of x^T likewise.  From the dequantized
    per-tensor rows (a given scale), x' = fl32(value(q) * s) is the float64
    product rounded once to binary32 (exact products of two binary32 values
    fit float64), and the 128x128 columns are the block quantizer of x'^T."""
    x = workloads.block_act(256, 384, seed=28)
    am = oracle.amax(x)
    h = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_PER_TENSOR, E4, oracle.SUBQ_MXFP8, E5, amax_in=am, margin=1)
    r = oracle.quantize_tensor(x, E4, amax_in=am, margin=1)
    qm, sm = oracle.quantize_mx_colwise(x, E5)
    assert np.array_equal(h["q_row"], r["q"]) and h["s_row"].tolist() == [r["scale_inv"]]
    assert np.array_equal(h["q_col"], qm) and np.array_equal(h["s_col"], sm)
    h = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_BLOCK_1x128, E4, oracle.SUBQ_PER_TENSOR, E5, amax_in=am)
    c = oracle.quantize_tensor(oracle.transpose(x), E5, amax_in=am)
    assert np.array_equal(h["q_col"], c["q"]) and h["s_col"].tolist() == [c["scale_inv"]]
    assert np.array_equal(h["q_row"], oracle.quantize_blocks(x, E4, 1, 128)[0])
    s = np.float32(0.0037)
    h = oracle.quantize_hybrid_blockwise(x, oracle.SUBQ_PER_TENSOR, E4, oracle.SUBQ_BLOCK_128x128, E4,
                                         oracle.COLSRC_ROWWISE_DEQUANTIZED, scale_inv_in=s)
    xp = (oracle.decode_table(E4)[h["q_row"]] * np.float64(s)).astype(np.float32)
    q_ref, s_ref = oracle.quantize_blocks(np.ascontiguousarray(xp.T), E4, 128, 128)
    assert np.array_equal(h["q_col"], q_ref) and np.array_equal(h["s_col"], s_ref)


def test_hybrid_rowwise_dequantized_is_idempotent_in_one_format():
    """Quantize, dequantize, quantize again with the same format and scale
    gives the same codes (the FP8 grid is far coarser than one fp32 rounding
    of value * s * (1/s)), so with equal given scales q_col = q_row^T; with a
    coarser column format it equals the E5M2 cast of the dequantized values,
    which differs from the cast of the original somewhere."""
    x = workloads.delayed_step(5, 128, 256)
    for s in (np.float32(0.3), np.float32(1 / 448), np.float32(2.0 ** -9)):
        h = oracle.quantize_hybrid(x, E4, E4, oracle.COLSRC_ROWWISE_DEQUANTIZED, row_scale_inv_in=s,
                                   col_scale_inv_in=s)
        assert np.array_equal(h["q_col"], oracle.transpose(h["q_row"]))
    s = np.float32(oracle.amax(x) / 448)
    d = oracle.quantize_hybrid(x, E4, E5, oracle.COLSRC_ROWWISE_DEQUANTIZED, row_scale_inv_in=s, col_scale_inv_in=s)
    o = oracle.quantize_hybrid(x, E4, E5, oracle.COLSRC_ORIGINAL, row_scale_inv_in=s, col_scale_inv_in=s)
    assert np.array_equal(d["q_row"], o["q_row"])
    xd = oracle.dequantize(d["q_row"], E4, s)
    assert np.array_equal(d["q_col"], oracle.transpose(oracle.quantize(xd, E5, oracle.reciprocal(s))))
    assert not np.array_equal(d["q_col"], o["q_col"])


def test_hybrid_dequantized_source_takes_its_own_amax():
    """Current scaling of the columnwise copy from the dequantized rowwise
    values uses max |x'|: with margin 2 the rowwise cast maps the largest
    element to 448 / 4 = 112 (exact in E4M3), so max |x'| = fl32(112 * s_r)."""
    x = np.float32([[3.0, -7.25, 0.5, 1.0] * 4] * 16)
    h = oracle.quantize_hybrid(x, E4, E5, oracle.COLSRC_ROWWISE_DEQUANTIZED, amax_in=np.float32(7.25),
                               row_margin=2, col_margin=0)
    s_r = np.float32(np.float32(7.25 / 448) * 4)
    assert f32_bits(h["row_scale_inv"]) == f32_bits(s_r)
    amax_d = np.float32(np.float32(112.0) * s_r)
    assert f32_bits(h["col_scale_inv"]) == f32_bits(np.float32(amax_d / np.float32(57344)))


def test_cast_stats_hand_cases():
    """E4M3 with s = 1: 449, 500 and +inf exceed 448 (3 overflows; -448 does
    not); 2^-10 (a tie, to the even zero) and 3e-4 become zero codes while
    2^-10 * 1.1 rounds up to 2^-9 (2 underflows); one NaN; 0 and -0 are not
    counted as nonzero."""
    x = np.float32([0.0, -0.0, 449, 500, -448, np.inf, 2.0 ** -10, 3e-4, 1.1 * 2.0 ** -10, np.nan, 1.0, -2.5])
    st = oracle.cast_stats(x, E4, 1.0)
    assert st.tolist() == [3, 2, 1, 9]
    # E5M2 reaches 57344 and 2^-16: with s = 1/64 the values are multiplied by 64
    st = oracle.cast_stats(np.float32([900.0, 896.0, 2.0 ** -23, 2.0 ** -22]), E5, 1 / 64)
    assert st.tolist() == [1, 1, 0, 4]


def test_cast_stats_counts_against_the_encoder():
    """On every bf16 pattern at three scales: overflows are the products
    (formed in float64, exact, and rounded once to float32) beyond FP8_MAX,
    and underflows the nonzero finite inputs that the pinned cast maps to a
    zero code."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = oracle._as_f32(bits)
    for fmt in (E4, E5):
        for s in (1.0, 1e-3, 37.5):
            st = oracle.cast_stats(bits, fmt, s)
            with np.errstate(over="ignore", invalid="ignore"):
                y = np.float32(xf.astype(np.float64) * float(oracle.reciprocal(s)))
            fin = np.isfinite(xf)
            assert st[2] == np.isnan(xf).sum()
            assert st[0] == (~np.isnan(xf) & (np.abs(y) > oracle.fmax(fmt))).sum()
            zero_code = (oracle.quantize(bits, fmt, oracle.reciprocal(s)) & 0x7F) == 0
            assert st[1] == (fin & (xf != 0) & zero_code).sum()


def _fp8_ulp(y: np.ndarray, fmt: int) -> np.ndarray:
    """Spacing of the FP8 grid at |y| from the bit layout (bias, mantissa bits)."""
    bias, mbits = (7, 3) if fmt == E4 else (15, 2)
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -40)))
    return 2.0 ** (np.maximum(e, 1 - bias) - mbits)


def test_error_feedback_telescopes_and_stays_below_half_a_step():
    """"Megatron FP8", section 25: with the residual carried over, the sum of
    what was sent plus the last residual equals the sum of the inputs (up to
    the fp32 roundings of v and of the residual, one ulp of |v| each per
    step), and each residual is at most half an FP8 step of its value."""
    rng = np.random.default_rng(3)
    n, T, s = 4096, 24, np.float32(2.0 ** -12)
    r = np.zeros(n, np.float32)
    sent = np.zeros(n, np.float64)
    total = np.zeros(n, np.float64)
    slack = np.zeros(n, np.float64)
    for t in range(T):
        g = workloads.to_bf16_bits(rng.standard_normal(n) * 1e-3 * (1 + t % 3))
        q, r_new, am = oracle.quantize_error_feedback(g, r, E5, s)
        v = oracle._as_f32(g).astype(np.float64) + r.astype(np.float64)
        assert am == np.float32(np.max(np.abs(np.float32(v))))
        dq = oracle.dequantize(q, E5, s).astype(np.float64)
        y = np.float32(v) * float(oracle.reciprocal(s))
        assert np.all(np.abs(r_new) <= 0.5 * _fp8_ulp(y, E5) * float(s) * (1 + 2.0 ** -20))
        sent += dq
        total += oracle._as_f32(g)
        slack += 2.0 ** -23 * np.abs(v)
        r = r_new
    assert np.all(np.abs(sent + r - total) <= 2 * slack)
