// quant.hip -- gfx950 kernels for the FP8 quantization side of the hot path:
// amax reduction, per-tensor scaled cast (optionally with the input amax
// fused in), dequantization, the delayed-scaling update, the rowwise +
// columnwise cast and block quantization.
//
// All element kernels are HBM-bound streams: 16-byte loads and stores per
// lane, several loads in flight per lane, and a VALU budget of a few
// instructions per element (the hardware converter does the rounding).
//
// Pages cited (title, section):
//   "Megatron FP8": section 2 (formats), 4 (scaling factors), 5 (delayed
//   scaling), 10 (margin), 23 (round-to-nearest-even);
//   "[Pytorch][Common] Hybrid quantization #2817" (rowwise/columnwise storage);
//   "Low Precision Training and Rollout" (128x128 block FP8, FP32 scales).
#include "fp8q_device.h"
#include "fp8q_launch.h"

namespace fp8q {

constexpr int kThreads = 256;

__host__ __device__ static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Flat streaming launches: the work is cut into units of kThreads * U
// vectors; block b takes units b, b + G, b + 2G, ... of a grid of
// G = min(units, kMaxGrid) blocks (one unit per block at the sizes of
// interest, so each lane issues its U loads back to back and the grid covers
// the chip many times over).
static int flat_grid(int64_t units)
{
    if (units < 1) return 1;
    return (int)(units < kMaxGrid ? units : kMaxGrid);
}

// The grid of a launch that reduces into the scratch: one partial slot per
// block, at most `cap` <= kParts blocks.  Fewer, longer-lived blocks leave
// fewer partials to fold at the end; measured on the MI355X over
// 8192x8192 bf16, a 1024-block cast with fused amax takes 38.8 us against
// 40.2 us at 2048 blocks and 46.8 us at 8192, and the read-only amax pass is
// fastest at 512 blocks (22.4 us, 23.2 us at 1024), where each lane still has
// four 16-byte loads in flight per unit.  With the finishing block that polls
// tagged slots, the delayed step (one launch) took 37.7 us per step with 1024
// producing blocks, 38.6 with 4096 and 46.8 with 8192 (slots enlarged to
// match), although the plain cast is fastest with one unit per block.
static int reduce_grid(int64_t units, int cap = kParts)
{
    if (units < 1) return 1;
    return (int)(units < cap ? units : cap);
}
constexpr int kAmaxGrid = kParts / 2;

template <int F>
__device__ __forceinline__ Scales resolve_scales(const ScaleSrc &src)
{
    if (src.amax_in) return current_scales(*src.amax_in, Fmt<F>::kMax, src.margin);
    return given_scales(*src.scale_inv_in);
}

__global__ void fill_u32_kernel(uint32_t *p, uint32_t v)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, hipStream_t s)
{
    fill_u32_kernel<<<1, 64, 0, s>>>(p, v);
    return hipGetLastError();
}

// One block's magnitude max -> its slot: published with the call's tag for
// the launch's finishing block (tag != 0), or stored to part[] for a finish
// kernel (tag 0).  Every lane must reach it.  The launch has at most kParts
// producing blocks.
__device__ __forceinline__ void block_partial(uint32_t m, GridScratch *gs, uint32_t tag)
{
    __shared__ uint32_t red[kThreads / 64];
    m = block_max_u32<kThreads>(m, red);
    if (threadIdx.x == 0) {
        if (tag) publish_partial(&gs->pub[blockIdx.x], tag, canonical_amax_bits(m));
        else gs->part[blockIdx.x] = canonical_amax_bits(m);
    }
}

// Read partial slot i and put it back to zero (one round trip).
__device__ __forceinline__ uint32_t take_partial(GridScratch *gs, int i) { return atomicExch(&gs->part[i], 0u); }

// Max of partial slots [0, nparts), which it leaves zero; kThreads lanes with
// up to kParts / kThreads exchanges in flight each.  Every lane gets the result.
__device__ __forceinline__ uint32_t take_partials(GridScratch *gs, int nparts)
{
    __shared__ uint32_t red[kThreads / 64];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < kParts / kThreads; ++u) {
        const int i = threadIdx.x + u * kThreads;
        if (i < nparts) m = max(m, take_partial(gs, i));
    }
    return block_max_u32<kThreads>(m, red);
}


// Delayed-scaling update ("Megatron FP8", section 5): write the step's amax
// at slot step % L of column col of the ring hist[L][n_cols], reduce the
// column (max, NaN-propagating; algo 0) or take the value just written (algo
// 1), and derive s = eff / FP8_MAX * 2^margin (1 when eff is not > 0) and its
// reciprocal for the column's next cast.  L may be any length.
struct DelayedUpdate {
    float *hist; // null: no update
    int L, n_cols, col, slot;
    float fmax;
    int margin, algo;
    float *scale, *scale_inv;
};

// Order-preserving key of a float for an unsigned max (negative values flip
// all bits, positive values set the sign bit); every NaN maps above +inf, so
// a NaN anywhere in the column wins the max.
__device__ __forceinline__ uint32_t order_key(float h)
{
    const uint32_t b = __float_as_uint(h);
    if (h != h) return 0xFFFFFFFFu;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The largest key of the column other than the slot being overwritten; a
// block of kThreads lanes, every lane gets it.
__device__ __forceinline__ uint32_t ring_key(const DelayedUpdate &d)
{
    __shared__ uint32_t red[kThreads / 64];
    uint32_t key = 0;
    for (int j = threadIdx.x; j < d.L; j += kThreads)
        if (j != d.slot) key = max(key, order_key(d.hist[(int64_t)j * d.n_cols + d.col]));
    return block_max_u32<kThreads>(key, red);
}

// One lane: record amax a and write the column's new scales.
__device__ __forceinline__ void ring_update(const DelayedUpdate &d, float a, uint32_t key)
{
    d.hist[(int64_t)d.slot * d.n_cols + d.col] = a;
    key = max(key, order_key(a));
    float eff;
    if (d.algo == 0)
        eff = key == 0xFFFFFFFFu ? __uint_as_float(kCanonicalNaN)
                                 : __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
    else
        eff = a;
    const float sv = (eff > 0.0f) ? ldexpf(eff / d.fmax, d.margin) : 1.0f;
    d.scale_inv[d.col] = sv;
    d.scale[d.col] = 1.0f / sv;
}

// What the finishing block of a reducing launch does with the amax: publish
// it (amax_out, canonical bits) and, for a delayed-scaling step, record it in
// the ring.  A launch has a finishing block when either is set.
// tag, rounds: the call's tag and polling bound (Reduce).
struct Finish {
    uint32_t *amax_out;
    DelayedUpdate du;
    uint32_t tag, rounds;
    __device__ __host__ bool active() const { return amax_out != nullptr || du.hist != nullptr; }
};

static Finish finish_amax_to(float *amax_out, const Reduce &r)
{
    return Finish{reinterpret_cast<uint32_t *>(amax_out), DelayedUpdate{}, r.tag, r.rounds};
}

__device__ __forceinline__ void finish_block(const Finish &f, GridScratch *gs, int nparts)
{
    // the ring is read while the producers still run
    const uint32_t key = f.du.hist ? ring_key(f.du) : 0u;
    const uint32_t a = collect_partials<kThreads, kParts>(gs->pub, nparts, f.tag, f.rounds);
    if (threadIdx.x == 0) {
        if (f.amax_out) *f.amax_out = a;
        if (f.du.hist) ring_update(f.du, __uint_as_float(a), key);
    }
}

__global__ __launch_bounds__(kThreads) void finish_amax_kernel(GridScratch *__restrict__ gs, int nparts,
                                                               uint32_t *__restrict__ out)
{
    const uint32_t m = take_partials(gs, nparts);
    if (threadIdx.x == 0) *out = m;
}

hipError_t launch_finish_amax(GridScratch *gs, int nparts, float *out, hipStream_t s)
{
    finish_amax_kernel<<<1, kThreads, 0, s>>>(gs, nparts, reinterpret_cast<uint32_t *>(out));
    return hipGetLastError();
}

__global__ __launch_bounds__(kThreads) void clear_scratch_kernel(GridScratch *__restrict__ gs)
{
    for (int i = threadIdx.x; i < kParts; i += kThreads) gs->part[i] = 0u;
    if (threadIdx.x < kStats * kCntParts) gs->cnt[threadIdx.x / kCntParts][threadIdx.x % kCntParts] = 0ull;
}

hipError_t launch_clear_scratch(GridScratch *gs, hipStream_t s)
{
    static_assert(kStats * kCntParts <= kThreads, "one lane per count slot");
    clear_scratch_kernel<<<1, kThreads, 0, s>>>(gs);
    return hipGetLastError();
}

// ---------------------------------------------------------- clock monitor --
// One wave per block measures the graphics clock of the CU it shares with
// other work: it reads the shader-clock counter (s_memtime, counts the CU's
// clock) and the constant-rate counter (s_memrealtime), then polls the stop
// word with agent-scope loads (which see a store made by a kernel that has
// finished on any XCD), sleeping briefly between polls, until the word is
// nonzero or `max_ticks` constant-rate ticks have passed (so the loop always
// ends), and reads both counters again.  Lanes 0, 1, 2 store the XCD id
// (HW_REG_XCC_ID bits 3:0) and the two deltas; block 0's lane 3 stores the
// constant rate in kHz.  Stores are per-lane vector stores.
__global__ __launch_bounds__(64) void clock_monitor_kernel(uint64_t *__restrict__ out, const uint32_t *stop,
                                                           uint64_t wall_khz, uint64_t max_ticks)
{
    const uint64_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        if (__builtin_amdgcn_s_memrealtime() - r0 >= max_ticks) break;
        __builtin_amdgcn_s_sleep(1);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x;
    const uint64_t v = lane == 0 ? xcc : lane == 1 ? t1 - t0 : lane == 2 ? r1 - r0 : wall_khz;
    if (lane < 3 || (lane == 3 && blockIdx.x == 0)) out[lane < 3 ? 3 * blockIdx.x + lane : 3 * kClockBlocks] = v;
}

hipError_t launch_clock_monitor(uint64_t *out, const uint32_t *stop, hipStream_t s)
{
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return e;
    if (khz <= 0) return hipErrorInvalidValue;
    // at most kClockMonitorSeconds of the constant-rate counter
    clock_monitor_kernel<<<kClockBlocks, 64, 0, s>>>(out, stop, (uint64_t)khz,
                                                     (uint64_t)khz * 1000 * kClockMonitorSeconds);
    return hipGetLastError();
}

// ------------------------------------------------------------------ amax --
// amax = max |x| ("Megatron FP8", section 4).  Each lane reads U 16-byte
// vectors of its unit, kThreads vectors apart (so every load instruction of a
// wave covers 1 KiB contiguously); the tail of fewer than one vector is read
// by the first lanes of block 0.
//
// An amax is read to scale the same tensor's cast (current scaling), which
// reads x again right after it.  The last kAmaxCacheKeep bytes of the input
// are therefore loaded without the non-temporal hint, so that the 256 MB
// last-level cache still holds them when the cast reads them; everything
// before them streams.  Measured on the MI355X, fp8_amax then
// fp8_quantize_tensor(amax_in) on 8192x8192 bf16 inputs rotating over 1 GiB:
// 57.3 us with every load streaming, 54.0 with the last 32 MiB kept, 52.6
// with 64 MiB and 51.6 with all 128 MiB; the amax alone takes 21.6, 21.2,
// 22.3 and 23.1 us.  (The cast's L2 hits, misses and fetched bytes are those
// of a cast of a cold input: the second read is served beyond the L2.)  The
// pair is what the method runs (the delayed recipe fuses its amax into the
// cast), so it is the one optimised.
#ifndef FP8Q_AMAX_U
#define FP8Q_AMAX_U 4
#endif
constexpr int kAmaxU = FP8Q_AMAX_U;
#ifndef FP8Q_AMAX_CACHE_KEEP_MIB
#define FP8Q_AMAX_CACHE_KEEP_MIB 128
#endif
constexpr int64_t kAmaxCacheKeep = (int64_t)FP8Q_AMAX_CACHE_KEEP_MIB << 20;

// The launch's last block is the finishing block, which writes the amax.
template <int DT>
__global__ __launch_bounds__(kThreads) void amax_kernel(const void *__restrict__ x, int64_t n, GridScratch *gs,
                                                        Finish fin)
{
    const int nwork = gridDim.x - 1;
    if (blockIdx.x == nwork) {
        finish_block(fin, gs, nwork);
        return;
    }
    constexpr int kPer = DT == kBF16 ? 8 : 4; // elements per 16-byte vector
    const int64_t nvec = n / kPer;
    const int64_t units = ceil_div(nvec, (int64_t)kThreads * kAmaxU);
    const uint4 *__restrict__ xv = reinterpret_cast<const uint4 *>(x);
    // units from `kept` on are loaded without the streaming hint
    const int64_t kept = units - kAmaxCacheKeep / (kThreads * kAmaxU * 16);
    uint32_t m = 0;
    u16x2 m2 = {0, 0};
    for (int64_t unit = blockIdx.x; unit < units; unit += nwork) {
        const int64_t base = unit * kThreads * kAmaxU + threadIdx.x;
        // lanes past the end re-read the last vector (harmless for a max)
        uint4 v[kAmaxU];
        if (unit < kept) {
#pragma unroll
            for (int u = 0; u < kAmaxU; ++u) {
                const int64_t i = base + u * kThreads;
                v[u] = ld_stream(xv + (i < nvec ? i : nvec - 1));
            }
        } else {
#pragma unroll
            for (int u = 0; u < kAmaxU; ++u) {
                const int64_t i = base + u * kThreads;
                v[u] = xv[i < nvec ? i : nvec - 1];
            }
        }
#pragma unroll
        for (int u = 0; u < kAmaxU; ++u) {
            if constexpr (DT == kBF16) {
                m2 = bf16_absmax2(m2, v[u].x);
                m2 = bf16_absmax2(m2, v[u].y);
                m2 = bf16_absmax2(m2, v[u].z);
                m2 = bf16_absmax2(m2, v[u].w);
            } else {
                m = max(m, v[u].x & 0x7FFFFFFFu);
                m = max(m, v[u].y & 0x7FFFFFFFu);
                m = max(m, v[u].z & 0x7FFFFFFFu);
                m = max(m, v[u].w & 0x7FFFFFFFu);
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < n - nvec * kPer) {
        const int64_t e = nvec * kPer + threadIdx.x;
        if constexpr (DT == kBF16)
            m = max(m, ((uint32_t)(reinterpret_cast<const uint16_t *>(x)[e] & 0x7FFFu)) << 16);
        else
            m = max(m, reinterpret_cast<const uint32_t *>(x)[e] & 0x7FFFFFFFu);
    }
    if constexpr (DT == kBF16) m = max(m, bf16_absmax_to_f32bits(m2));
    block_partial(m, gs, fin.tag);
}

hipError_t launch_amax(const void *x, int dtype, int64_t n, float *amax, const Reduce &r, hipStream_t s)
{
    const int64_t nvec = n / (dtype == kBF16 ? 8 : 4);
    // the producing blocks and the finishing block
    const int grid = reduce_grid(ceil_div(nvec, (int64_t)kThreads * kAmaxU), kAmaxGrid) + 1;
    const Finish fin = finish_amax_to(amax, r);
    if (dtype == kBF16)
        amax_kernel<kBF16><<<grid, kThreads, 0, s>>>(x, n, r.gs, fin);
    else
        amax_kernel<kF32><<<grid, kThreads, 0, s>>>(x, n, r.gs, fin);
    return hipGetLastError();
}

// ------------------------------------------------------------------ cast --
// Load 16 consecutive elements (one chunk) as floats (streaming loads unless
// the caller asks for plain ones).
template <int DT> struct Chunk16;
template <> struct Chunk16<kBF16> {
    uint32_t w[8]; // 16 bf16
    template <bool kNT = true> __device__ __forceinline__ void load(const void *x, int64_t c)
    {
        const uint4 *p = reinterpret_cast<const uint4 *>(x) + 2 * c;
        const uint4 a = kNT ? ld_stream(p) : p[0], b = kNT ? ld_stream(p + 1) : p[1];
        w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w, w[4] = b.x, w[5] = b.y, w[6] = b.z, w[7] = b.w;
    }
    __device__ __forceinline__ float get(int k) const { return (k & 1) ? bf16_hi(w[k >> 1]) : bf16_lo(w[k >> 1]); }
    __device__ __forceinline__ void absmax(uint32_t &, u16x2 &m2) const
    {
#pragma unroll
        for (int j = 0; j < 8; ++j) m2 = bf16_absmax2(m2, w[j]);
    }
};
template <> struct Chunk16<kF32> {
    uint32_t w[16]; // 16 floats
    template <bool kNT = true> __device__ __forceinline__ void load(const void *x, int64_t c)
    {
        const uint4 *p = reinterpret_cast<const uint4 *>(x) + 4 * c;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 v = kNT ? ld_stream(p + j) : p[j];
            w[4 * j] = v.x, w[4 * j + 1] = v.y, w[4 * j + 2] = v.z, w[4 * j + 3] = v.w;
        }
    }
    __device__ __forceinline__ float get(int k) const { return __uint_as_float(w[k]); }
    __device__ __forceinline__ void absmax(uint32_t &m, u16x2 &) const
    {
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, w[j] & 0x7FFFFFFFu);
    }
};

template <int F, int DT>
__device__ __forceinline__ uint4 encode_chunk(const Chunk16<DT> &c, float scale)
{
    uint4 o;
    o.x = encode4<F>(c.get(0), c.get(1), c.get(2), c.get(3), scale);
    o.y = encode4<F>(c.get(4), c.get(5), c.get(6), c.get(7), scale);
    o.z = encode4<F>(c.get(8), c.get(9), c.get(10), c.get(11), scale);
    o.w = encode4<F>(c.get(12), c.get(13), c.get(14), c.get(15), scale);
    return o;
}

// --------------------------------------------------------- cast statistics --
// Diagnostics of a per-tensor cast ("Megatron FP8", section 24: per-tensor
// overflow and underflow counts next to amax and scale).  With
// y = fl32(x * fl32(1/s)):
//   overflow  -- x not NaN and |y| > FP8_MAX (the cast saturates it);
//   underflow -- x finite and nonzero and its code a zero code, i.e. |y| at
//                most half the smallest subnormal (the tie rounds to the even
//                zero): |y| <= 2^-10 (E4M3FN) or 2^-17 (E5M2);
//   NaN, and nonzero (not NaN, x != 0).
// |y| is monotone in |x|, so the classes are intervals of the magnitude bits
// m of x: zero, underflow (0, U], normal, overflow (O, inf], NaN above inf,
// with U and O the largest magnitudes whose products stay at or below the
// limits (found per block by a short walk from limit / scale, a bisection over
// the bit patterns only if the walk does not settle).  A lane counts m > T
// for T = 0, U, O, inf and the four counts follow by differences.  bf16
// magnitudes are 16-bit, two to a register, and m > T is the sign bit of the
// packed 16-bit difference T - m; fp32 magnitudes take the sign of T - m.
// fp8_cast_stats is a read-only stream like the amax, and the cast can count
// in its own pass; either way each block writes four partial counts and a
// one-block kernel sums them into 64-bit totals.
template <int F> struct Tiny;
template <> struct Tiny<kE4M3> { static constexpr float kHalfMinSub = 0x1p-10f; };
template <> struct Tiny<kE5M2> { static constexpr float kHalfMinSub = 0x1p-17f; };

// Largest magnitude bits m in [0, 0x7F800000] with |fl32(m * scale)| <= limit
// (0 when even the smallest nonzero magnitude exceeds it).  The answer lies
// within a few patterns of limit / |scale|: a short walk from there, checked
// at both ends, and a bisection only if the walk does not settle (every
// block runs this once, so it must cost far less than its stream).
__device__ __forceinline__ bool within(uint32_t m, float scale, float limit)
{
    return fabsf(__uint_as_float(m) * scale) <= limit;
}

__device__ __forceinline__ uint32_t last_magnitude_within(float scale, float limit)
{
    uint32_t c = min(f32_absbits(limit / scale), kInfBits);
#pragma unroll
    for (int i = 0; i < 4 && c < kInfBits && within(c + 1, scale, limit); ++i) ++c;
#pragma unroll
    for (int i = 0; i < 4 && c > 0 && !within(c, scale, limit); ++i) --c;
    if ((c == 0 || within(c, scale, limit)) && (c == kInfBits || !within(c + 1, scale, limit))) return c;
    uint32_t lo = 0, hi = kInfBits;
    if (within(hi, scale, limit)) return hi;
    while (hi - lo > 1) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (within(mid, scale, limit)) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Thresholds T[0..3] = 0, U, O, inf (magnitude bits).
template <int F> __device__ __forceinline__ void stat_thresholds(float scale, uint32_t T[kStats])
{
    T[0] = 0;
    T[3] = kInfBits;
    if (scale != scale) { // NaN products: neither overflow nor underflow
        T[1] = 0;
        T[2] = kInfBits;
    } else {
        T[1] = last_magnitude_within(scale, Tiny<F>::kHalfMinSub);
        // with a zero scale inf * 0 is NaN: nothing overflows
        T[2] = scale == 0.0f ? kInfBits : last_magnitude_within(scale, Fmt<F>::kMax);
    }
}

// Per-block counts of m > T[k] -> partials of (overflows, underflows, NaNs,
// nonzeros).
__device__ __forceinline__ void block_counts(const uint32_t g[kStats], GridScratch *gs)
{
    __shared__ uint32_t red[kStats][kThreads / 64];
    const uint32_t c[kStats] = {g[2] - g[3], g[0] - g[1], g[3], g[0] - g[3]};
#pragma unroll
    for (int k = 0; k < kStats; ++k) {
        uint32_t v = c[k];
        // wave sum with DPP row shifts and broadcasts (total in lane 63)
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
        if ((threadIdx.x & 63) == 63) red[k][threadIdx.x >> 6] = v;
    }
    __syncthreads();
    if (threadIdx.x < kStats) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) t += red[threadIdx.x][w];
        if (t) atomicAdd(&gs->cnt[threadIdx.x][blockIdx.x % kCntParts], (unsigned long long)t);
    }
}

// Add the counts m > T[k] of one chunk to g.
__device__ __forceinline__ void chunk_counts(const Chunk16<kBF16> &c, const uint32_t T[kStats], uint32_t g[kStats])
{
    // 16-bit magnitudes: m16 << 16 > T  <=>  m16 > T >> 16, and with both
    // below 2^15 that is the sign bit of the 16-bit difference T16 - m16
#pragma unroll
    for (int k = 0; k < kStats; ++k) {
        const u16x2 t = {(unsigned short)(T[k] >> 16), (unsigned short)(T[k] >> 16)};
        u16x2 acc = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += (u16x2)((t - as_u16x2(c.w[j] & 0x7FFF7FFFu)) >> (unsigned short)15);
        g[k] += (uint32_t)acc.x + (uint32_t)acc.y;
    }
}

__device__ __forceinline__ void chunk_counts(const Chunk16<kF32> &c, const uint32_t T[kStats], uint32_t g[kStats])
{
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t m = c.w[j] & 0x7FFFFFFFu;
#pragma unroll
        for (int k = 0; k < kStats; ++k) g[k] += (T[k] - m) >> 31; // m, T < 2^31
    }
}

// Per-tensor cast ("Megatron FP8", section 4): q = encode(fl32(x * scale)).
// Every lane derives the scale from the device scalar (no host round trip);
// block 0 publishes it.  A lane encodes U chunks of 16 elements of its unit,
// kThreads chunks apart, into one 16-byte store each.  With kAmax the input's
// magnitude max is reduced in the same pass into the block's partial
// (delayed scaling records it after the cast, section 5).  With kCount the
// same pass counts the cast's overflows, underflows, NaNs and nonzeros
// (section 24) against the scale it casts with.
#ifndef FP8Q_CAST_U
#define FP8Q_CAST_U 2
#endif
constexpr int kCastU = FP8Q_CAST_U;

template <int F, int DT, bool kAmax, bool kCount = false>
__global__ __launch_bounds__(kThreads) void cast_kernel(const void *__restrict__ x, int64_t n, ScaleSrc src,
                                                        uint8_t *__restrict__ q, float *scale_inv_out,
                                                        float *scale_out, GridScratch *gs, Finish fin)
{
    // with a finisher (kAmax only) the launch's last block finishes the call
    const int nwork = gridDim.x - (kAmax && fin.active() ? 1 : 0);
    if (kAmax && blockIdx.x == nwork) {
        finish_block(fin, gs, nwork);
        return;
    }
    const Scales sc = resolve_scales<F>(src);
    uint32_t T[kStats], g[kStats] = {0, 0, 0, 0};
    if constexpr (kCount) stat_thresholds<F>(sc.scale, T);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (scale_inv_out) *scale_inv_out = sc.s;
        if (scale_out) *scale_out = sc.scale;
    }
    const int64_t nch = n >> 4;
    const int64_t units = ceil_div(nch, (int64_t)kThreads * kCastU);
    uint4 *__restrict__ qv = reinterpret_cast<uint4 *>(q);
    uint32_t m = 0;
    u16x2 m2 = {0, 0};
    for (int64_t unit = blockIdx.x; unit < units; unit += nwork) {
        const int64_t base = unit * kThreads * kCastU + threadIdx.x;
        // Lanes past the end re-read the last chunk (a valid address, so all
        // loads are unconditional and stay in registers) and store nothing;
        // re-reading an element does not change a max.
        Chunk16<DT> c[kCastU];
#pragma unroll
        for (int u = 0; u < kCastU; ++u) {
            const int64_t ci = base + u * kThreads;
            c[u].load(x, ci < nch ? ci : nch - 1);
        }
#pragma unroll
        for (int u = 0; u < kCastU; ++u) {
            if constexpr (kAmax) c[u].absmax(m, m2);
            const uint4 o = encode_chunk<F, DT>(c[u], sc.scale);
            if (base + u * kThreads < nch) {
                st_stream(qv + base + u * kThreads, o);
                if constexpr (kCount) chunk_counts(c[u], T, g); // a re-read chunk must not count twice
            }
        }
    }
    // tail: fewer than 16 elements, one per lane of block 0
    if (blockIdx.x == 0 && threadIdx.x < n - (nch << 4)) {
        const int64_t e = (nch << 4) + threadIdx.x;
        float v;
        if constexpr (DT == kBF16)
            v = __uint_as_float(((uint32_t)reinterpret_cast<const uint16_t *>(x)[e]) << 16);
        else
            v = reinterpret_cast<const float *>(x)[e];
        if constexpr (kAmax) m = max(m, f32_absbits(v));
        q[e] = (uint8_t)encode1<F>(v, sc.scale);
        if constexpr (kCount) {
#pragma unroll
            for (int k = 0; k < kStats; ++k) g[k] += f32_absbits(v) > T[k] ? 1u : 0u;
        }
    }
    if constexpr (kAmax) {
        if constexpr (DT == kBF16) m = max(m, bf16_absmax_to_f32bits(m2));
        block_partial(m, gs, fin.active() ? fin.tag : 0u);
    }
    if constexpr (kCount) block_counts(g, gs);
}

static hipError_t launch_finish_stats(GridScratch *gs, uint64_t *stats, hipStream_t s);

template <int F, int DT>
static hipError_t launch_cast_t(const void *x, int64_t n, ScaleSrc src, uint8_t *q, float *scale_inv_out,
                                float *scale_out, float *amax_out, uint64_t *stats, const Reduce &r, hipStream_t s)
{
    const int64_t units = ceil_div(n >> 4, (int64_t)kThreads * kCastU);
    const int grid = (amax_out || stats) ? reduce_grid(units) : flat_grid(units);
    const Finish none{nullptr, DelayedUpdate{}, 0u, 0u};
    if (stats) {
        // the counts are summed by the statistics kernel, which follows
        if (amax_out)
            cast_kernel<F, DT, true, true><<<grid, kThreads, 0, s>>>(x, n, src, q, scale_inv_out, scale_out, r.gs,
                                                                     none);
        else
            cast_kernel<F, DT, false, true><<<grid, kThreads, 0, s>>>(x, n, src, q, scale_inv_out, scale_out, r.gs,
                                                                      none);
    } else if (amax_out) {
        // the producing blocks and the finishing block, which writes the amax
        cast_kernel<F, DT, true><<<grid + 1, kThreads, 0, s>>>(x, n, src, q, scale_inv_out, scale_out, r.gs,
                                                                finish_amax_to(amax_out, r));
    } else {
        cast_kernel<F, DT, false><<<grid, kThreads, 0, s>>>(x, n, src, q, scale_inv_out, scale_out, nullptr, none);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && stats && amax_out) e = launch_finish_amax(r.gs, grid, amax_out, s);
    if (e == hipSuccess && stats) e = launch_finish_stats(r.gs, stats, s);
    return e;
}

hipError_t launch_cast(const void *x, int dtype, int64_t n, int fmt, ScaleSrc src, uint8_t *q, float *scale_inv_out,
                       float *scale_out, float *amax_out, uint64_t *stats, const Reduce &r, hipStream_t s)
{
    if (fmt == kE4M3) {
        if (dtype == kBF16)
            return launch_cast_t<kE4M3, kBF16>(x, n, src, q, scale_inv_out, scale_out, amax_out, stats, r, s);
        return launch_cast_t<kE4M3, kF32>(x, n, src, q, scale_inv_out, scale_out, amax_out, stats, r, s);
    }
    if (dtype == kBF16)
        return launch_cast_t<kE5M2, kBF16>(x, n, src, q, scale_inv_out, scale_out, amax_out, stats, r, s);
    return launch_cast_t<kE5M2, kF32>(x, n, src, q, scale_inv_out, scale_out, amax_out, stats, r, s);
}

// --------------------------------------------------------------- dequant --
template <int F, bool kHi>
__device__ __forceinline__ float2 dec2(uint32_t w)
{
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f r;
    if constexpr (F == kE4M3)
        r = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
    else
        r = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, kHi);
    return make_float2(r.x, r.y);
}

// y = fl32(value(q) * scale_inv) ("Megatron FP8", section 4).  The hardware
// decoder gives the exact value of every code.  A lane decodes U words of
// four codes, kThreads words apart, each into one 16-byte store, so that every
// store instruction of a wave writes 1 KiB contiguously (the output is four
// times the input and dominates the traffic).
constexpr int kDequantU = 2;

template <int F>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t *__restrict__ q, int64_t n,
                                                           const float *__restrict__ scale_inv, float *__restrict__ y)
{
    const float s = *scale_inv;
    const int64_t nw = n >> 2;
    const int64_t units = ceil_div(nw, (int64_t)kThreads * kDequantU);
    const uint32_t *__restrict__ qw = reinterpret_cast<const uint32_t *>(q);
    float4 *__restrict__ yv = reinterpret_cast<float4 *>(y);
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int64_t base = unit * kThreads * kDequantU + threadIdx.x;
        uint32_t w[kDequantU];
#pragma unroll
        for (int u = 0; u < kDequantU; ++u) {
            const int64_t i = base + u * kThreads;
            w[u] = ld_stream_u32(qw + (i < nw ? i : nw - 1));
        }
#pragma unroll
        for (int u = 0; u < kDequantU; ++u) {
            const float2 lo = dec2<F, false>(w[u]);
            const float2 hi = dec2<F, true>(w[u]);
            if (base + u * kThreads < nw)
                st_stream(yv + base + u * kThreads, make_uint4(__float_as_uint(lo.x * s), __float_as_uint(lo.y * s),
                                                               __float_as_uint(hi.x * s), __float_as_uint(hi.y * s)));
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < n - (nw << 2)) {
        const int64_t e = (nw << 2) + threadIdx.x;
        y[e] = dec2<F, false>((uint32_t)q[e]).x * s;
    }
}

hipError_t launch_dequant(const uint8_t *q, int fmt, int64_t n, const float *scale_inv, float *y, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const int grid = flat_grid(ceil_div(n >> 2, (int64_t)kThreads * kDequantU));
    if (fmt == kE4M3)
        dequant_kernel<kE4M3><<<grid, kThreads, 0, s>>>(q, n, scale_inv, y);
    else
        dequant_kernel<kE5M2><<<grid, kThreads, 0, s>>>(q, n, scale_inv, y);
    return hipGetLastError();
}

constexpr int kStatsU = 4;

template <int F, int DT>
__global__ __launch_bounds__(kThreads) void cast_stats_kernel(const void *__restrict__ x, int64_t n,
                                                              const float *__restrict__ scale_inv, GridScratch *gs)
{
    uint32_t T[kStats];
    stat_thresholds<F>(1.0f / *scale_inv, T);
    const int64_t nch = n >> 4;
    const int64_t units = ceil_div(nch, (int64_t)kThreads * kStatsU);
    uint32_t g[kStats] = {0, 0, 0, 0};
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int64_t base = unit * kThreads * kStatsU + threadIdx.x;
        Chunk16<DT> ch[kStatsU];
#pragma unroll
        for (int u = 0; u < kStatsU; ++u) {
            const int64_t ci = base + u * kThreads;
            ch[u].load(x, ci < nch ? ci : nch - 1);
        }
#pragma unroll
        for (int u = 0; u < kStatsU; ++u) // counts, unlike a max, must not see a chunk twice
            if (base + u * kThreads < nch) chunk_counts(ch[u], T, g);
    }
    if (blockIdx.x == 0 && threadIdx.x < n - (nch << 4)) {
        const int64_t e = (nch << 4) + threadIdx.x;
        uint32_t m;
        if constexpr (DT == kBF16)
            m = ((uint32_t)reinterpret_cast<const uint16_t *>(x)[e] & 0x7FFFu) << 16;
        else
            m = reinterpret_cast<const uint32_t *>(x)[e] & 0x7FFFFFFFu;
#pragma unroll
        for (int k = 0; k < kStats; ++k) g[k] += m > T[k] ? 1u : 0u;
    }
    block_counts(g, gs);
}

// One wave per statistic: lane i takes count slot i (and zeroes it), the
// wave sums them into the 64-bit total.
__global__ __launch_bounds__(kStats * kCntParts) void finish_stats_kernel(GridScratch *__restrict__ gs,
                                                                          uint64_t *__restrict__ out)
{
    static_assert(kCntParts == 64, "one wave per statistic");
    const int k = threadIdx.x >> 6;
    uint64_t v = atomicExch(&gs->cnt[k][threadIdx.x & 63], 0ull);
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) out[k] = v;
}

hipError_t launch_cast_stats(const void *x, int dtype, int64_t n, int fmt, const float *scale_inv, uint64_t *stats,
                             GridScratch *gs, hipStream_t s)
{
    const int grid = reduce_grid(ceil_div(n >> 4, (int64_t)kThreads * kStatsU));
    if (fmt == kE4M3) {
        if (dtype == kBF16) cast_stats_kernel<kE4M3, kBF16><<<grid, kThreads, 0, s>>>(x, n, scale_inv, gs);
        else cast_stats_kernel<kE4M3, kF32><<<grid, kThreads, 0, s>>>(x, n, scale_inv, gs);
    } else {
        if (dtype == kBF16) cast_stats_kernel<kE5M2, kBF16><<<grid, kThreads, 0, s>>>(x, n, scale_inv, gs);
        else cast_stats_kernel<kE5M2, kF32><<<grid, kThreads, 0, s>>>(x, n, scale_inv, gs);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_finish_stats(gs, stats, s);
}

static hipError_t launch_finish_stats(GridScratch *gs, uint64_t *stats, hipStream_t s)
{
    finish_stats_kernel<<<1, kStats * kCntParts, 0, s>>>(gs, stats);
    return hipGetLastError();
}

// --------------------------------------------------------- error feedback --
// One step of FP8 quantization with error feedback ("Megatron FP8", section
// 25): v = fl32(g + r), q = encode(fl32(v * fl32(1/s))), and the residual
// keeps what the cast lost, r = fl32(v - fl32(value(q) * s)), for the next
// step; the amax of v is reduced in the same pass (delayed scaling records it).
// A lane handles U chunks of 16 elements: the residual is read and written by
// the same lane, so the in-place update needs no synchronisation.
constexpr int kEfU = 2;

template <int F, int DT>
__global__ __launch_bounds__(kThreads) void error_feedback_kernel(const void *__restrict__ g,
                                                                  float *__restrict__ residual, int64_t n,
                                                                  const float *__restrict__ scale_inv,
                                                                  uint8_t *__restrict__ q, GridScratch *gs,
                                                                  Finish fin)
{
    // v - value * s is rounded twice (product, then difference), as defined:
    // no fused multiply-add
#pragma clang fp contract(off)
    // with an amax the launch's last block is the finishing block
    const bool amax = fin.active();
    const int nwork = gridDim.x - (amax ? 1 : 0);
    if (amax && blockIdx.x == nwork) {
        finish_block(fin, gs, nwork);
        return;
    }
    const float s = *scale_inv;
    const float scale = 1.0f / s;
    const int64_t nch = n >> 4;
    const int64_t units = ceil_div(nch, (int64_t)kThreads * kEfU);
    float4 *__restrict__ rv = reinterpret_cast<float4 *>(residual);
    uint4 *__restrict__ qv = reinterpret_cast<uint4 *>(q);
    uint32_t m = 0;
    for (int64_t unit = blockIdx.x; unit < units; unit += nwork) {
        const int64_t base = unit * kThreads * kEfU + threadIdx.x;
        Chunk16<DT> ch[kEfU];
        float4 r[kEfU][4];
#pragma unroll
        for (int u = 0; u < kEfU; ++u) {
            const int64_t ci = base + u * kThreads;
            const int64_t cc = ci < nch ? ci : nch - 1;
            // plain loads: with the residual updated in place, streaming
            // hints on this kernel's accesses measured slower, not faster
            ch[u].template load<false>(g, cc);
#pragma unroll
            for (int j = 0; j < 4; ++j) r[u][j] = rv[4 * cc + j];
        }
#pragma unroll
        for (int u = 0; u < kEfU; ++u) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[4 * j] = ch[u].get(4 * j) + r[u][j].x;
                v[4 * j + 1] = ch[u].get(4 * j + 1) + r[u][j].y;
                v[4 * j + 2] = ch[u].get(4 * j + 2) + r[u][j].z;
                v[4 * j + 3] = ch[u].get(4 * j + 3) + r[u][j].w;
            }
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = encode4<F>(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], scale);
            if (base + u * kThreads < nch) {
                const int64_t ci = base + u * kThreads;
                qv[ci] = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float2 lo = dec2<F, false>(w[j]), hi = dec2<F, true>(w[j]);
                    rv[4 * ci + j] = make_float4(v[4 * j] - lo.x * s, v[4 * j + 1] - lo.y * s,
                                                 v[4 * j + 2] - hi.x * s, v[4 * j + 3] - hi.y * s);
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) m = max(m, f32_absbits(v[k]));
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < n - (nch << 4)) {
        const int64_t e = (nch << 4) + threadIdx.x;
        float gv;
        if constexpr (DT == kBF16)
            gv = __uint_as_float(((uint32_t)reinterpret_cast<const uint16_t *>(g)[e]) << 16);
        else
            gv = reinterpret_cast<const float *>(g)[e];
        const float v = gv + residual[e];
        const uint32_t c = encode1<F>(v, scale);
        q[e] = (uint8_t)c;
        residual[e] = v - dec2<F, false>(c).x * s;
        m = max(m, f32_absbits(v));
    }
    if (amax) block_partial(m, gs, fin.tag);
}

hipError_t launch_error_feedback(const void *g, int dtype, float *residual, int64_t n, int fmt,
                                 const float *scale_inv, uint8_t *q, float *amax_out, const Reduce &r, hipStream_t s)
{
    const Finish am = finish_amax_to(amax_out, r);
    GridScratch *gs = r.gs;
    const int64_t units = ceil_div(n >> 4, (int64_t)kThreads * kEfU);
    // with an amax: the producing blocks and the finishing block
    const int grid = amax_out ? reduce_grid(units) + 1 : flat_grid(units);
    if (fmt == kE4M3) {
        if (dtype == kBF16) error_feedback_kernel<kE4M3, kBF16><<<grid, kThreads, 0, s>>>(g, residual, n, scale_inv, q, gs, am);
        else error_feedback_kernel<kE4M3, kF32><<<grid, kThreads, 0, s>>>(g, residual, n, scale_inv, q, gs, am);
    } else {
        if (dtype == kBF16) error_feedback_kernel<kE5M2, kBF16><<<grid, kThreads, 0, s>>>(g, residual, n, scale_inv, q, gs, am);
        else error_feedback_kernel<kE5M2, kF32><<<grid, kThreads, 0, s>>>(g, residual, n, scale_inv, q, gs, am);
    }
    return hipGetLastError();
}

// --------------------------------------------------------------- delayed --
// The standalone update (fp8_update_delayed): the new amax is read from
// memory; one block records it and derives the column's scales.
__global__ __launch_bounds__(kThreads) void delayed_kernel(DelayedUpdate d, const float *__restrict__ new_amax)
{
    const uint32_t key = ring_key(d);
    if (threadIdx.x == 0) ring_update(d, *new_amax, key);
}

static float fmax_of(int fmt) { return fmt == kE4M3 ? Fmt<kE4M3>::kMax : Fmt<kE5M2>::kMax; }

static DelayedUpdate make_update(float *hist, int history_len, int n_cols, int col, int64_t step, int fmt, int margin,
                                 int algo, float *scale, float *scale_inv)
{
    return DelayedUpdate{hist, history_len, n_cols, col, (int)(step % history_len), fmax_of(fmt), margin, algo,
                         scale, scale_inv};
}

hipError_t launch_delayed(float *hist, int history_len, int n_cols, int col, const float *new_amax, int64_t step,
                          int fmt, int margin, int algo, float *scale, float *scale_inv, hipStream_t s)
{
    delayed_kernel<<<1, kThreads, 0, s>>>(make_update(hist, history_len, n_cols, col, step, fmt, margin, algo, scale,
                                                      scale_inv),
                                          new_amax);
    return hipGetLastError();
}

// One delayed-scaling step, one launch: the cast of x with the stored scale of
// column col (scale_inv[col]) reduces the input's amax into per-block
// partials, and the launch's finishing block folds them, publishes the amax
// and updates the ring and the column's scales for the format of the next
// step.  The scale it overwrites is read by every casting block at its start,
// before that block publishes its partial, so no block of this launch casts
// with the next step's scale.
hipError_t launch_delayed_step(const void *x, int dtype, int64_t n, int fmt, float *hist, int history_len, int n_cols,
                               int col, int64_t step, int fmt_next, int margin, int algo, float *scale,
                               float *scale_inv, uint8_t *q, float *q_scale_inv_out, float *amax_out, const Reduce &r,
                               hipStream_t s)
{
    const ScaleSrc src{nullptr, scale_inv + col, 0};
    GridScratch *gs = r.gs;
    const Finish fin{reinterpret_cast<uint32_t *>(amax_out),
                     make_update(hist, history_len, n_cols, col, step, fmt_next, margin, algo, scale, scale_inv),
                     r.tag, r.rounds};
    const int grid = reduce_grid(ceil_div(n >> 4, (int64_t)kThreads * kCastU)) + 1;
    if (fmt == kE4M3) {
        if (dtype == kBF16)
            cast_kernel<kE4M3, kBF16, true><<<grid, kThreads, 0, s>>>(x, n, src, q, q_scale_inv_out, nullptr, gs, fin);
        else
            cast_kernel<kE4M3, kF32, true><<<grid, kThreads, 0, s>>>(x, n, src, q, q_scale_inv_out, nullptr, gs, fin);
    } else {
        if (dtype == kBF16)
            cast_kernel<kE5M2, kBF16, true><<<grid, kThreads, 0, s>>>(x, n, src, q, q_scale_inv_out, nullptr, gs, fin);
        else
            cast_kernel<kE5M2, kF32, true><<<grid, kThreads, 0, s>>>(x, n, src, q, q_scale_inv_out, nullptr, gs, fin);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------- tile kernels --
// A 128x128 tile per block of 256 lanes.  Lane (ig = tid / 8, jg = tid % 8)
// owns rows 4*ig .. 4*ig+3 and columns 16*jg .. 16*jg+15 of the tile: four
// rows of 16 elements, read as 16-byte vectors and written as one 16-byte
// vector of codes per row (8 lanes cover a 128-byte row segment).
//
// The columnwise copy goes through LDS: each lane transposes its 4x16 codes
// in registers (byte permutes) into 16 dwords, one per column, each holding
// four consecutive rows; the dwords land in LDS as a [128 col][128 row] byte
// tile, rotated by 8 dwords per 16 columns so that the writes of a wave spread
// over all banks while every 16-byte read stays contiguous.
// kTileHybrid + colF + 2 * dequantized_source: per-direction per-tensor
// quantization (row codes in format F, column codes in format colF with their
// own scale, from x or from the dequantized row codes).
//
// tile_kernel<F, DT, kMode, kAmax, FCol, kColMode, kColDeq>: the row codes by
// the recipe kMode in format F; the column codes in format FCol by the recipe
// kColMode (by default the row recipe, so the single-recipe modes above are
// tile_kernel<F, DT, kMode, kAmax>), from x or, with kColDeq, from the
// dequantized row codes.  A pass quantizes each direction with its own block
// maxima; at most one of the two directions is per-tensor when they differ.
enum TileMode { kTilePerTensor = 0, kTileBlock128 = 1, kTileBlock1x128 = 2, kTileMX = 3, kTileHybrid = 4 };

// MXFP8 shared scale of one 32-element block from its magnitude max (float
// bits, NaN above 0x7F800000): e = floor(log2(amax)) - emax clamped to
// [-127, 127] (emax = 8 for E4M3FN, 15 for E5M2; 0 gives -127, Inf gives 127),
// the E8M0 byte e + 127 (255 for NaN) and the exact multiplier 2^-e.
struct MxScale {
    float mult;
    uint32_t byte;
};

template <int F> __device__ __forceinline__ MxScale mx_scale(uint32_t abits)
{
    constexpr int emax = F == kE4M3 ? 8 : 15;
    if (abits > kInfBits) return {__uint_as_float(kCanonicalNaN), 255u};
    int e;
    if (abits == 0) {
        e = -127;
    } else if (abits == kInfBits) {
        e = 127;
    } else {
        const int biased = (int)(abits >> 23);
        const int fl = biased ? biased - 127 : (31 - __builtin_clz(abits)) - 149; // floor(log2)
        e = min(max(fl - emax, -127), 127);
    }
    // 2^-e: a normal float for -e >= -126, the subnormal 2^-127 for e = 127
    const uint32_t mbits = e < 127 ? (uint32_t)(127 - e) << 23 : 0x00400000u;
    return {__uint_as_float(mbits), (uint32_t)(e + 127)};
}

// Value of an E8M0 scale byte: 2^(b - 127) (2^-127 is a subnormal), NaN for 255.
__device__ __forceinline__ float e8m0_value(uint32_t b)
{
    if (b == 255u) return __uint_as_float(kCanonicalNaN);
    return __uint_as_float(b ? b << 23 : 0x00400000u);
}

constexpr int kTile = 128;

// 4x4 byte transpose: d[r] holds row r (bytes = columns 0..3); e[c] returns
// column c (bytes = rows 0..3).
__device__ __forceinline__ void transpose4x4(const uint32_t d0, const uint32_t d1, const uint32_t d2,
                                             const uint32_t d3, uint32_t e[4])
{
    const uint32_t lo01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u); // d0.b0 d1.b0 d0.b1 d1.b1
    const uint32_t hi01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u); // d0.b2 d1.b2 d0.b3 d1.b3
    const uint32_t lo23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
    e[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    e[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    e[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    e[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// dword address in the transposed LDS tile of (tile column j, row dword d).
// A column is 32 dwords, so two columns fill the 64 banks.  The rotation by 8
// dwords per 16 columns spreads the 8 lanes jg = 0..7 of one staging write
// over 32 banks; swapping the two columns of a pair when bit 6 of j is set
// puts lanes jg >= 4 on the other 32, so the 64 lanes of a write hit 64
// distinct banks.  Every 16-byte read stays contiguous.
__device__ __forceinline__ int tlds_addr(int j, int d)
{
    return (j ^ ((j >> 6) & 1)) * 32 + ((d + 8 * (j >> 4)) & 31);
}

// A lane's 4 rows x 16 columns of input as raw 16-byte vectors.
template <int DT> struct RawPatch {
    static constexpr int kVec = DT == kBF16 ? 2 : 4; // 16-byte vectors per row
    uint4 w[4][kVec];
    template <bool kNT> __device__ __forceinline__ void load(const void *x, int64_t ld, int64_t r0, int64_t c0)
    {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(x) +
                                                             ((r0 + r) * ld + c0) * (DT == kBF16 ? 2 : 4));
#pragma unroll
            for (int k = 0; k < kVec; ++k) w[r][k] = kNT ? ld_stream(p + k) : p[k];
        }
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k = 0; k < kVec; ++k) w[r][k] = make_uint4(0, 0, 0, 0);
    }
};

// Hide a raw patch's words from the optimiser, so that floats derived from
// it before this point are recomputed after it instead of being kept live.
template <int DT> __device__ __forceinline__ void opaque(RawPatch<DT> &p)
{
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int k = 0; k < RawPatch<DT>::kVec; ++k) {
            uint32_t a = p.w[r][k].x, b = p.w[r][k].y, c = p.w[r][k].z, d = p.w[r][k].w;
            asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
            p.w[r][k] = make_uint4(a, b, c, d);
        }
}

// Element (r, k) of a raw patch as a float (k is a compile-time constant in
// every use, so this is one shift or mask for bf16 and nothing for fp32; the
// floats are recomputed where needed rather than kept across the barriers).
template <int DT>
__device__ __forceinline__ float patch_elem(const RawPatch<DT> &p, int r, int k)
{
    if constexpr (DT == kBF16) {
        const uint4 a = p.w[r][k >> 3];
        const int e = (k & 7) >> 1;
        const uint32_t w = e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w;
        return (k & 1) ? bf16_hi(w) : bf16_lo(w);
    } else {
        const uint4 a = p.w[r][k >> 2];
        const int e = k & 3;
        return __uint_as_float(e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w);
    }
}

// Magnitude maxima (fp32 bit patterns, NaN above 0x7F800000) of the lane's
// 4 x 16 patch: per row of 16 elements and per column of 4.  bf16 words hold
// two elements, maximised together with packed 16-bit operations.
template <int DT> __device__ __forceinline__ uint32_t patch_word(const RawPatch<DT> &p, int r, int j)
{
    const uint4 a = p.w[r][j >> 2];
    const int e = j & 3;
    return e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w;
}

template <int DT> __device__ __forceinline__ void patch_row_max(const RawPatch<DT> &p, uint32_t row[4])
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (DT == kBF16) {
            u16x2 m = as_u16x2(patch_word<DT>(p, r, 0) & 0x7FFF7FFFu);
#pragma unroll
            for (int j = 1; j < 8; ++j) m = __builtin_elementwise_max(m, as_u16x2(patch_word<DT>(p, r, j) & 0x7FFF7FFFu));
            row[r] = bf16_absmax_to_f32bits(m);
        } else {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) m = max(m, patch_word<DT>(p, r, j) & 0x7FFFFFFFu);
            row[r] = m;
        }
    }
}

template <int DT> __device__ __forceinline__ void patch_col_max(const RawPatch<DT> &p, uint32_t col[16])
{
    if constexpr (DT == kBF16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { // word j holds columns 2j (low half) and 2j + 1
            u16x2 m = as_u16x2(patch_word<DT>(p, 0, j) & 0x7FFF7FFFu);
#pragma unroll
            for (int r = 1; r < 4; ++r) m = __builtin_elementwise_max(m, as_u16x2(patch_word<DT>(p, r, j) & 0x7FFF7FFFu));
            col[2 * j] = (uint32_t)m.x << 16;
            col[2 * j + 1] = (uint32_t)m.y << 16;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            uint32_t m = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) m = max(m, patch_word<DT>(p, r, k) & 0x7FFFFFFFu);
            col[k] = m;
        }
    }
}

template <bool B> struct Rep {
    static constexpr bool value = B;
};

// Store the lane's 4x16 codes (cw[r][0..3] = row r, 16 codes) transposed into LDS.
__device__ __forceinline__ void stage_transposed(uint32_t *tl, const uint32_t cw[4][4], int ig, int jg)
{
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        uint32_t e[4];
        transpose4x4(cw[0][q4], cw[1][q4], cw[2][q4], cw[3][q4], e);
#pragma unroll
        for (int k = 0; k < 4; ++k) tl[tlds_addr(jg * 16 + q4 * 4 + k, ig)] = e[k];
    }
}

// Write the transposed tile from LDS to q_col [cols][rows]: output row
// (tile column j), 16 consecutive rows k*16 .. k*16+15 per 16-byte store.
template <bool kNT>
__device__ __forceinline__ void store_transposed(const uint32_t *tl, uint8_t *q_col, int64_t rows, int64_t cols,
                                                 int64_t row0, int64_t col0)
{
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int p = threadIdx.x + u * kThreads;
        const int j = p >> 3, k = p & 7;
        if (col0 + j < cols && row0 + 16 * k < rows) {
            const uint4 v = *reinterpret_cast<const uint4 *>(tl + tlds_addr(j, 4 * k));
            if constexpr (kNT) st_stream(q_col + (col0 + j) * rows + row0 + 16 * k, v);
            else *reinterpret_cast<uint4 *>(q_col + (col0 + j) * rows + row0 + 16 * k) = v;
        }
    }
}

// One block loops over tiles t = blockIdx.x, blockIdx.x + G, ... (tile row
// t / tiles_per_row, tile column t % tiles_per_row), G the number of tile
// blocks (with kAmax the launch has one more, its finishing block).
template <int F, int DT, int kMode, bool kAmax, int FCol = F, int kColMode = kMode, bool kColDeq = false>
__global__ __launch_bounds__(kThreads) void tile_kernel(const void *__restrict__ x, int64_t rows, int64_t cols,
                                                        ScaleSrc src, uint8_t *__restrict__ q_row,
                                                        uint8_t *__restrict__ q_col, void *__restrict__ s_row_p,
                                                        void *__restrict__ s_col_p, float *scale_inv_out,
                                                        float *scale_out, GridScratch *gs, ScaleSrc src_col,
                                                        float *col_scale_inv_out, Finish fin)
{
    // with kAmax the launch's last block is the finishing block
    const int nwork = gridDim.x - (kAmax ? 1 : 0);
    if (kAmax && blockIdx.x == nwork) {
        finish_block(fin, gs, nwork);
        return;
    }
    constexpr bool kHybrid = kMode >= kTileHybrid;
    constexpr int FC = kHybrid ? ((kMode - kTileHybrid) & 1) : FCol; // format of the column codes
    constexpr bool kDeq = kHybrid && ((kMode - kTileHybrid) >> 1); // columns from the dequantized rows
    // the block recipe of the column codes (kColMode) may differ from that
    // of the row codes (kMode): each direction's scales come from its own
    // block maxima, taken over x or, with kColDeq, over the dequantized row
    // values x' = fl32(value(row code) * d), d the row block's dequant scale
    constexpr bool kRow128 = kMode == kTileBlock128;
    constexpr bool kCol128 = kColMode == kTileBlock128, kCol1x = kColMode == kTileBlock1x128,
                   kColMX = kColMode == kTileMX;
    // block scales: fp32 (128x128, 1x128) or E8M0 bytes (MXFP8)
    float *__restrict__ s_row = reinterpret_cast<float *>(s_row_p);
    float *__restrict__ s_col = reinterpret_cast<float *>(s_col_p);
    uint8_t *__restrict__ e_row = reinterpret_cast<uint8_t *>(s_row_p);
    uint8_t *__restrict__ e_col = reinterpret_cast<uint8_t *>(s_col_p);
    __shared__ uint32_t tl[kTile * 32]; // transposed codes, 16 KiB
    __shared__ uint32_t red[kThreads / 64];
    __shared__ uint32_t colmax[kCol1x ? 4 * kTile : 1]; // per wave, per tile column
    __shared__ float colscale[kCol1x ? kTile : 1];
    __shared__ uint32_t ecol[kColMX ? kTile : 1]; // MXFP8: a tile column's 4 scale bytes
    __shared__ uint32_t colbad; // 1x128: some column scale of the tile is NaN, infinite or zero

    const int ig = threadIdx.x >> 3, jg = threadIdx.x & 7;
    const int64_t tiles_c = ceil_div(cols, kTile), tiles = tiles_c * ceil_div(rows, kTile);
    const int64_t brows = rows / kTile, bcols = cols / kTile; // block-scale grid (block modes)

    Scales sc_tensor{1.0f, 1.0f}, sc_col{1.0f, 1.0f};
    if constexpr (kMode == kTilePerTensor || kHybrid) {
        sc_tensor = resolve_scales<F>(src);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (scale_inv_out) *scale_inv_out = sc_tensor.s;
            if (scale_out) *scale_out = sc_tensor.scale;
        }
    }
    if constexpr (kHybrid) {
        if (kDeq && src_col.amax_in) {
            // current scaling of the dequantized rows: their amax is the
            // image of amax(x) under the (monotone) cast and dequantization
            const uint32_t c = encode1<F>(*src_col.amax_in, sc_tensor.scale);
            sc_col = current_scales(dec2<F, false>(c).x * sc_tensor.s, Fmt<FC>::kMax, src_col.margin);
        } else {
            sc_col = resolve_scales<FC>(src_col);
        }
        if (blockIdx.x == 0 && threadIdx.x == 0 && col_scale_inv_out) *col_scale_inv_out = sc_col.s;
    }
    // per-tensor column codes under a block recipe of the rows
    constexpr bool kColTensor = kColMode == kTilePerTensor && kMode != kTilePerTensor;
    if constexpr (kColTensor) {
        sc_col = resolve_scales<FC>(src_col);
        if (blockIdx.x == 0 && threadIdx.x == 0 && col_scale_inv_out) *col_scale_inv_out = sc_col.s;
    }
    uint32_t m_all = 0; // per-tensor fused amax

    // Cache hints, chosen per mode by measurement on the MI355X (unlike the
    // flat kernels, a tile kernel's 128-byte row pieces and transposed
    // columns do not all gain from the non-temporal hint): the per-tensor
    // cast streams its loads and its column stores (8192x8192 bf16 55.3 ->
    // 54.2 us), the block modes stream their column stores (128x128 blocks of
    // 7168x4096 25.6 -> 24.5 us, 1x128 blocks of 4096x7168 30.5 -> 29.9 us),
    // and the MXFP8 and per-direction modes, slower with either hint, keep
    // plain accesses; streamed loads alone made the per-tensor cast 13%
    // slower, and streamed row stores slowed every mode.
    constexpr bool kNTLoad = kMode == kTilePerTensor;
    constexpr bool kNTColStore = kColMode == kTilePerTensor || kCol128 || kCol1x;

    // The lane's patch of tile t (rows % 4 == 0 and cols % 16 == 0, so a patch
    // is either whole or entirely outside the matrix).
    auto load_patch = [&](int64_t t, RawPatch<DT> &raw) {
        const int64_t tr = t / tiles_c, tc = t - tr * tiles_c;
        const int64_t r0 = tr * kTile + 4 * ig, c0 = tc * kTile + 16 * jg;
        if (r0 < rows && c0 < cols) raw.template load<kNTLoad>(x, cols, r0, c0);
        else raw.zero();
    };
    for (int64_t t = blockIdx.x; t < tiles; t += nwork) {
        const int64_t tr = t / tiles_c, tc = t - tr * tiles_c;
        const int64_t row0 = tr * kTile, col0 = tc * kTile;
        const int64_t r0 = row0 + 4 * ig, c0 = col0 + 16 * jg;
        const bool valid = (r0 < rows) && (c0 < cols);

        RawPatch<DT> p;
        load_patch(t, p);
#define PV(r, k) patch_elem<DT>(p, (r), (k))

        uint32_t cw[4][4]; // rowwise codes
        [[maybe_unused]] float dq[4]; // kColDeq: the dequant scale of each of the lane's rows
        // Encodes of the lane's 4 x 16 patch; kR selects the NaN-repairing
        // encode, needed only when some product can be NaN (a NaN input, or a
        // scale that is NaN, infinite or zero).  Every mode encodes with the
        // short form and, in that rare case alone, encodes again with repair
        // (one unconditional path keeps the two from sharing registers).
        auto enc_rows = [&](auto rep, float scale) {
            constexpr bool kR = decltype(rep)::value;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    cw[r][q4] = encode4<F, kR>(PV(r, 4 * q4), PV(r, 4 * q4 + 1), PV(r, 4 * q4 + 2), PV(r, 4 * q4 + 3),
                                               scale);
        };

        if constexpr (kMode == kTilePerTensor || kHybrid) {
            uint32_t rm[4];
            patch_row_max<DT>(p, rm);
            const uint32_t pmax = max(max(rm[0], rm[1]), max(rm[2], rm[3]));
            if constexpr (kAmax) m_all = max(m_all, pmax);
            enc_rows(Rep<false>{}, sc_tensor.scale);
            if (!(pmax <= kInfBits && finite_nonzero(sc_tensor.scale))) {
                opaque(p);
                enc_rows(Rep<true>{}, sc_tensor.scale);
            }
            if constexpr (kColDeq) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dq[r] = sc_tensor.s;
            }
        } else if constexpr (kMode == kTileBlock128) {
            uint32_t rm[4];
            patch_row_max<DT>(p, rm);
            uint32_t m = max(max(rm[0], rm[1]), max(rm[2], rm[3]));
            m = block_max_u32<kThreads>(m, red);
            const float amax_b = __uint_as_float(canonical_amax_bits(m));
            const Scales sc = current_scales(amax_b, Fmt<F>::kMax, 0);
            // 128x128 columns of x in a format of their own: the same block
            // amax, that format's scale (other column recipes, and columns of
            // x', set their scales below)
            if constexpr (kCol128 && FC != F && !kColDeq) sc_col = current_scales(amax_b, Fmt<FC>::kMax, 0);
            if constexpr (kColDeq) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dq[r] = sc.s;
            }
            if (threadIdx.x == 0) {
                if (q_row) s_row[tr * bcols + tc] = sc.s;
                if (kCol128 && !kColDeq && s_col) s_col[tc * brows + tr] = FC != F ? sc_col.s : sc.s;
            }
            // the block scale is uniform: finite and nonzero exactly when the
            // block holds no NaN or infinity
            enc_rows(Rep<false>{}, sc.scale);
            if (!finite_nonzero(sc.scale)) {
                opaque(p);
                enc_rows(Rep<true>{}, sc.scale);
            }
        } else if constexpr (kMode == kTileMX) {
            // MXFP8: 1x32 row blocks are two lanes (jg = 2b, 2b + 1) of a row;
            // 32x1 column blocks are the 8 lanes of one wave sharing jg (the
            // wave holds rows 32w .. 32w+31 of the tile), so no block scale
            // leaves its wave.  A block's multiplier is a finite, nonzero power
            // of two unless the block holds a NaN.
            const int64_t xrow = cols / 32;
            uint32_t rm[4];
            patch_row_max<DT>(p, rm);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t m = rm[r];
                m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false)); // lane ^ 1
                const MxScale ms = mx_scale<F>(m);
                if constexpr (kColDeq) dq[r] = e8m0_value(ms.byte);
                // the row's 4 scale bytes of this tile sit in lanes jg = 0, 2, 4, 6:
                // gather them into lane jg = 0 (row_shl:n reads lane + n) for one
                // 4-byte store instead of four byte stores
                const uint32_t b1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ms.byte, 0x102, 0xF, 0xF, false);
                const uint32_t b2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ms.byte, 0x104, 0xF, 0xF, false);
                const uint32_t b3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ms.byte, 0x106, 0xF, 0xF, false);
                if (jg == 0 && valid && q_row)
                    *reinterpret_cast<uint32_t *>(e_row + (r0 + r) * xrow + (col0 >> 5)) =
                        ms.byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    cw[r][q4] = encode4<F, false>(PV(r, 4 * q4), PV(r, 4 * q4 + 1), PV(r, 4 * q4 + 2),
                                                  PV(r, 4 * q4 + 3), ms.mult);
                if (m > kInfBits) {
                    opaque(p);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        cw[r][q4] = encode4<F, true>(PV(r, 4 * q4), PV(r, 4 * q4 + 1), PV(r, 4 * q4 + 2),
                                                     PV(r, 4 * q4 + 3), ms.mult);
                }
                if (q_row && valid)
                    *reinterpret_cast<uint4 *>(q_row + (r0 + r) * cols + c0) =
                        make_uint4(cw[r][0], cw[r][1], cw[r][2], cw[r][3]);
            }
        } else { // 1x128 blocks: one scale per row segment, one per column segment
            // row segments: the 8 lanes jg = 0..7 of a row group hold the row's 128 columns
            uint32_t rm[4];
            patch_row_max<DT>(p, rm);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t m = rm[r];
                m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false)); // lane ^ 1
                m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false)); // lane ^ 2
                // lane 7 - i of the 8 (DPP row_half_mirror): the other quad
                m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
                const Scales sc = current_scales(__uint_as_float(canonical_amax_bits(m)), Fmt<F>::kMax, 0);
                if constexpr (kColDeq) dq[r] = sc.s;
                if (jg == 0 && q_row) s_row[(r0 + r) * bcols + tc] = sc.s;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    cw[r][q4] = encode4<F, false>(PV(r, 4 * q4), PV(r, 4 * q4 + 1), PV(r, 4 * q4 + 2),
                                                  PV(r, 4 * q4 + 3), sc.scale);
                if (!finite_nonzero(sc.scale)) {
                    opaque(p);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        cw[r][q4] = encode4<F, true>(PV(r, 4 * q4), PV(r, 4 * q4 + 1), PV(r, 4 * q4 + 2),
                                                     PV(r, 4 * q4 + 3), sc.scale);
                }
                // stored now (unless the column codes come from them, the rowwise
                // codes need not stay live through the column phase)
                if (q_row && valid)
                    *reinterpret_cast<uint4 *>(q_row + (r0 + r) * cols + c0) =
                        make_uint4(cw[r][0], cw[r][1], cw[r][2], cw[r][3]);
            }
            opaque(p);
        }

        if (kMode != kTileBlock1x128 && kMode != kTileMX && q_row && valid) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<uint4 *>(q_row + (r0 + r) * cols + c0) =
                    make_uint4(cw[r][0], cw[r][1], cw[r][2], cw[r][3]);
        }

        // x'(r, k), the dequantized row value of the lane's element (r, k); the
        // repairing form gives a NaN x' (a NaN row code, or a zero code times
        // an infinite block scale) the sign of its row code
        auto xq = [&](auto rep, int r, int k) -> float {
            const uint32_t w = cw[r][k >> 2];
            const float2 h = (k & 2) ? dec2<F, true>(w) : dec2<F, false>(w);
            float v = ((k & 1) ? h.y : h.x) * dq[r];
            if constexpr (decltype(rep)::value) {
                if (v != v) v = __uint_as_float(kCanonicalNaN | (((w >> (8 * (k & 3))) & 0x80u) << 24));
            }
            return v;
        };
        // the value a column code is formed from: x, or x' with kColDeq
        auto cv = [&](auto rep, int r, int k) -> float {
            if constexpr (kColDeq) return xq(rep, r, k);
            else return PV(r, k);
        };
        // the lane's column maxima (magnitude bits) over its 4 rows
        auto col_max = [&](uint32_t cmx[16]) {
            if constexpr (kColDeq) {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    uint32_t m = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) m = max(m, __float_as_uint(xq(Rep<false>{}, r, k)) & 0x7FFFFFFFu);
                    cmx[k] = m;
                }
            } else {
                patch_col_max<DT>(p, cmx);
            }
        };

        // column scales of the block recipes (and, for MXFP8, the column codes)
        if constexpr (kColMX) {
            if (q_col) {
                opaque(p);
                uint32_t cmax[16];
                col_max(cmax);
                float cm[16];
                uint32_t cb[16], worst = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    uint32_t m = cmax[k];
                    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xF, 0xF, false)); // lane ^ 8
                    m = max_xor16(m);                                                                     // lane ^ 16
                    m = max_xor32(m);                                                                     // lane ^ 32
                    worst = max(worst, m);
                    const MxScale ms = mx_scale<FC>(m);
                    cm[k] = ms.mult;
                    cb[k] = ms.byte;
                }
                // a tile column's 4 scale bytes (one per wave) meet in LDS and
                // leave as one 4-byte store after the barrier below
                if ((threadIdx.x & 63) < 8) {
                    uint8_t *eb = reinterpret_cast<uint8_t *>(ecol);
#pragma unroll
                    for (int k = 0; k < 16; ++k) eb[(16 * jg + k) * 4 + (threadIdx.x >> 6)] = (uint8_t)cb[k];
                }
                uint32_t cc[4][4];
                auto enc_cols = [&](auto rep) {
                    constexpr bool kR = decltype(rep)::value;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int k = 4 * q4;
                            cc[r][q4] = encode4s<FC, kR>(cv(rep, r, k), cv(rep, r, k + 1), cv(rep, r, k + 2),
                                                         cv(rep, r, k + 3), cm[k], cm[k + 1], cm[k + 2], cm[k + 3]);
                        }
                };
                enc_cols(Rep<false>{});
                if (worst > kInfBits) {
                    opaque(p);
                    enc_cols(Rep<true>{});
                }
                stage_transposed(tl, cc, ig, jg);
            }
        } else if constexpr (kCol1x) {
            // column segments: a column's 128 rows are 4 rows in each of 32
            // lanes; the 8 of them in one wave (lane bits 3..5) are reduced
            // with cross-lane moves, the 4 waves through LDS
            if (q_col) {
                const int wv = threadIdx.x >> 6;
                uint32_t cm[16];
                col_max(cm);
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    uint32_t m = cm[k];
                    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xF, 0xF, false)); // lane ^ 8
                    m = max_xor16(m);                                                                     // lane ^ 16
                    m = max_xor32(m);                                                                     // lane ^ 32
                    cm[k] = m;
                }
                if ((threadIdx.x & 63) < 8) {
                    uint4 *dst = reinterpret_cast<uint4 *>(colmax + wv * kTile + 16 * jg);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        dst[q4] = make_uint4(cm[4 * q4], cm[4 * q4 + 1], cm[4 * q4 + 2], cm[4 * q4 + 3]);
                }
                if (threadIdx.x == 0) colbad = 0;
                __syncthreads();
                if (threadIdx.x < kTile) {
                    const uint32_t m = max(max(colmax[threadIdx.x], colmax[kTile + threadIdx.x]),
                                           max(colmax[2 * kTile + threadIdx.x], colmax[3 * kTile + threadIdx.x]));
                    const Scales sc = current_scales(__uint_as_float(canonical_amax_bits(m)), Fmt<FC>::kMax, 0);
                    colscale[threadIdx.x] = sc.scale;
                    s_col[(col0 + threadIdx.x) * brows + tr] = sc.s;
                    if (!finite_nonzero(sc.scale)) colbad = 1;
                }
                __syncthreads();
            }
        } else if constexpr (kCol128 && (!kRow128 || kColDeq)) {
            if (q_col) {
                uint32_t lm = 0;
                if constexpr (kColDeq) {
                    uint32_t cmx[16];
                    col_max(cmx);
#pragma unroll
                    for (int k = 0; k < 16; ++k) lm = max(lm, cmx[k]);
                } else {
                    uint32_t rm[4];
                    patch_row_max<DT>(p, rm);
                    lm = max(max(rm[0], rm[1]), max(rm[2], rm[3]));
                }
                const uint32_t m = block_max_u32<kThreads>(lm, red);
                sc_col = current_scales(__uint_as_float(canonical_amax_bits(m)), Fmt<FC>::kMax, 0);
                if (threadIdx.x == 0) s_col[tc * brows + tr] = sc_col.s;
            }
        }
        if (q_col) {
            if constexpr (kCol1x) {
                // columnwise codes use the column-segment scales
                opaque(p);
                uint32_t cc[4][4];
                auto enc_cols = [&](auto rep) {
                    constexpr bool kR = decltype(rep)::value;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int k = 4 * q4;
                            const float *cs = colscale + 16 * jg + k;
                            cc[r][q4] = encode4s<FC, kR>(cv(rep, r, k), cv(rep, r, k + 1), cv(rep, r, k + 2),
                                                         cv(rep, r, k + 3), cs[0], cs[1], cs[2], cs[3]);
                        }
                };
                enc_cols(Rep<false>{});
                if (colbad != 0) {
                    opaque(p);
                    enc_cols(Rep<true>{});
                }
                stage_transposed(tl, cc, ig, jg);
            } else if constexpr (kHybrid) {
                // column codes in their own format and scale, from x or from
                // x' = fl32(value(row code) * s_row)
                uint32_t rm[4];
                patch_row_max<DT>(p, rm);
                const bool clean = max(max(rm[0], rm[1]), max(rm[2], rm[3])) <= kInfBits &&
                                   finite_nonzero(sc_tensor.scale) && finite_nonzero(sc_col.scale) &&
                                   (!kDeq || finite_nonzero(sc_tensor.s));
                uint32_t cc[4][4];
                auto enc_cols = [&](auto rep) {
                    constexpr bool kR = decltype(rep)::value;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            if constexpr (kDeq) {
                                const uint32_t w = cw[r][q4];
                                const float2 lo = dec2<F, false>(w), hi = dec2<F, true>(w);
                                const float sr = sc_tensor.s;
                                const float d0 = lo.x * sr, d1 = lo.y * sr, d2 = hi.x * sr, d3 = hi.y * sr;
                                uint32_t c = encode4<FC, kR>(d0, d1, d2, d3, sc_col.scale);
                                if constexpr (kR) {
                                    // a NaN row code stays NaN with the sign of its code
                                    // (the decoder's NaN carries no sign of its own)
                                    if (__builtin_expect((d0 != d0) | (d1 != d1) | (d2 != d2) | (d3 != d3), 0)) {
                                        const uint32_t flip =
                                            ((__float_as_uint(sr) ^ __float_as_uint(sc_col.scale)) >> 24) & 0x80u;
                                        const float d[4] = {d0, d1, d2, d3};
#pragma unroll
                                        for (int b = 0; b < 4; ++b)
                                            if (d[b] != d[b])
                                                c = (c & ~(0xFFu << (8 * b))) |
                                                    ((0x7Fu | (((w >> (8 * b)) & 0x80u) ^ flip)) << (8 * b));
                                    }
                                }
                                cc[r][q4] = c;
                            } else {
                                cc[r][q4] = encode4<FC, kR>(PV(r, 4 * q4), PV(r, 4 * q4 + 1), PV(r, 4 * q4 + 2),
                                                            PV(r, 4 * q4 + 3), sc_col.scale);
                            }
                        }
                };
                enc_cols(Rep<false>{});
                if (!clean) {
                    opaque(p);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) asm volatile("" : "+v"(cw[r][q4]));
                    enc_cols(Rep<true>{});
                }
                stage_transposed(tl, cc, ig, jg);
            } else if constexpr (kCol128 && (FC != F || !kRow128 || kColDeq)) {
                // the block's column codes in their own format or recipe, from x or x'
                opaque(p);
                uint32_t cc[4][4];
                auto enc_cols = [&](auto rep) {
                    constexpr bool kR = decltype(rep)::value;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            cc[r][q4] = encode4<FC, kR>(cv(rep, r, 4 * q4), cv(rep, r, 4 * q4 + 1),
                                                        cv(rep, r, 4 * q4 + 2), cv(rep, r, 4 * q4 + 3), sc_col.scale);
                };
                enc_cols(Rep<false>{});
                if (!finite_nonzero(sc_col.scale)) {
                    opaque(p);
                    enc_cols(Rep<true>{});
                }
                stage_transposed(tl, cc, ig, jg);
            } else if constexpr (kColTensor) {
                // per-tensor column codes of x or x' with their own scale
                uint32_t cmx[16];
                col_max(cmx);
                uint32_t lm = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) lm = max(lm, cmx[k]);
                const bool clean = lm <= kInfBits && finite_nonzero(sc_col.scale);
                uint32_t cc[4][4];
                auto enc_cols = [&](auto rep) {
                    constexpr bool kR = decltype(rep)::value;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            cc[r][q4] = encode4<FC, kR>(cv(rep, r, 4 * q4), cv(rep, r, 4 * q4 + 1),
                                                        cv(rep, r, 4 * q4 + 2), cv(rep, r, 4 * q4 + 3), sc_col.scale);
                };
                enc_cols(Rep<false>{});
                if (!clean) {
                    opaque(p);
                    enc_cols(Rep<true>{});
                }
                stage_transposed(tl, cc, ig, jg);
            } else if constexpr (!kColMX) { // (MXFP8 staged its own column codes above)
                stage_transposed(tl, cw, ig, jg);
            }
            __syncthreads();
            store_transposed<kNTColStore>(tl, q_col, rows, cols, row0, col0);
            if constexpr (kColMX) {
                const int64_t xcol = rows / 32;
                if (threadIdx.x < kTile && col0 + threadIdx.x < cols)
                    *reinterpret_cast<uint32_t *>(e_col + (col0 + threadIdx.x) * xcol + (row0 >> 5)) =
                        ecol[threadIdx.x];
            }
        }
        __syncthreads(); // the next tile reuses the LDS buffers
#undef PV
    }
    if constexpr (kAmax) block_partial(m_all, gs, fin.tag);
}

static int tile_grid(int64_t rows, int64_t cols, bool reduce = false)
{
    const int64_t tiles = ceil_div(rows, kTile) * ceil_div(cols, kTile);
    return reduce ? reduce_grid(tiles) : flat_grid(tiles);
}

template <int F, int DT>
static hipError_t launch_rc_t(const void *x, int64_t rows, int64_t cols, ScaleSrc src, uint8_t *q_row, uint8_t *q_col,
                              float *scale_inv_out, float *scale_out, float *amax_out, const Reduce &r, hipStream_t s)
{
    // with an amax: the producing blocks and the finishing block
    const int grid = tile_grid(rows, cols, amax_out != nullptr) + (amax_out ? 1 : 0);
    if (amax_out)
        tile_kernel<F, DT, kTilePerTensor, true><<<grid, kThreads, 0, s>>>(
            x, rows, cols, src, q_row, q_col, nullptr, nullptr, scale_inv_out, scale_out, r.gs, ScaleSrc{}, nullptr,
            finish_amax_to(amax_out, r));
    else
        tile_kernel<F, DT, kTilePerTensor, false><<<grid, kThreads, 0, s>>>(x, rows, cols, src, q_row, q_col, nullptr,
                                                                           nullptr, scale_inv_out, scale_out, nullptr,
                                                                           ScaleSrc{}, nullptr, Finish{});
    return hipGetLastError();
}

hipError_t launch_rowwise_colwise(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, ScaleSrc src,
                                  uint8_t *q_row, uint8_t *q_col, float *scale_inv_out, float *scale_out,
                                  float *amax_out, const Reduce &r, hipStream_t s)
{
    if (rows == 0 || cols == 0) {
        // still publish the scales and an amax of 0
        return launch_cast(x, dtype, 0, fmt, src, nullptr, scale_inv_out, scale_out, amax_out, nullptr, r, s);
    }
    if (fmt == kE4M3) {
        if (dtype == kBF16)
            return launch_rc_t<kE4M3, kBF16>(x, rows, cols, src, q_row, q_col, scale_inv_out, scale_out, amax_out, r,
                                             s);
        return launch_rc_t<kE4M3, kF32>(x, rows, cols, src, q_row, q_col, scale_inv_out, scale_out, amax_out, r, s);
    }
    if (dtype == kBF16)
        return launch_rc_t<kE5M2, kBF16>(x, rows, cols, src, q_row, q_col, scale_inv_out, scale_out, amax_out, r, s);
    return launch_rc_t<kE5M2, kF32>(x, rows, cols, src, q_row, q_col, scale_inv_out, scale_out, amax_out, r, s);
}

template <int F, int DT, int kMode>
static hipError_t launch_hybrid_m(const void *x, int64_t rows, int64_t cols, ScaleSrc src, ScaleSrc src_col,
                                  uint8_t *q_row, uint8_t *q_col, float *row_scale_inv_out, float *col_scale_inv_out,
                                  float *amax_out, const Reduce &r, hipStream_t s)
{
    // with an amax: the producing blocks and the finishing block
    const int grid = tile_grid(rows, cols, amax_out != nullptr) + (amax_out ? 1 : 0);
    if (amax_out)
        tile_kernel<F, DT, kMode, true><<<grid, kThreads, 0, s>>>(x, rows, cols, src, q_row, q_col, nullptr, nullptr,
                                                                 row_scale_inv_out, nullptr, r.gs, src_col,
                                                                 col_scale_inv_out, finish_amax_to(amax_out, r));
    else
        tile_kernel<F, DT, kMode, false><<<grid, kThreads, 0, s>>>(x, rows, cols, src, q_row, q_col, nullptr, nullptr,
                                                                  row_scale_inv_out, nullptr, nullptr, src_col,
                                                                  col_scale_inv_out, Finish{});
    return hipGetLastError();
}

template <int F, int DT>
static hipError_t launch_hybrid_t(const void *x, int64_t rows, int64_t cols, int col_fmt, int col_source, ScaleSrc src,
                                  ScaleSrc src_col, uint8_t *q_row, uint8_t *q_col, float *row_scale_inv_out,
                                  float *col_scale_inv_out, float *amax_out, const Reduce &r, hipStream_t s)
{
    const int mode = kTileHybrid + col_fmt + 2 * col_source;
#define FP8Q_HYBRID(M)                                                                                              \
    case M:                                                                                                         \
        return launch_hybrid_m<F, DT, M>(x, rows, cols, src, src_col, q_row, q_col, row_scale_inv_out,              \
                                         col_scale_inv_out, amax_out, r, s)
    switch (mode) {
        FP8Q_HYBRID(kTileHybrid);
        FP8Q_HYBRID(kTileHybrid + 1);
        FP8Q_HYBRID(kTileHybrid + 2);
        FP8Q_HYBRID(kTileHybrid + 3);
    }
#undef FP8Q_HYBRID
    return hipErrorInvalidValue;
}

hipError_t launch_hybrid(const void *x, int dtype, int64_t rows, int64_t cols, int row_fmt, int col_fmt,
                         int col_source, ScaleSrc src, ScaleSrc src_col, uint8_t *q_row, uint8_t *q_col,
                         float *row_scale_inv_out, float *col_scale_inv_out, float *amax_out, const Reduce &r,
                         hipStream_t s)
{
    // an empty tensor still publishes both scales and an amax of 0: the grid
    // is one block with no tiles to visit
#define FP8Q_ARGS x, rows, cols, col_fmt, col_source, src, src_col, q_row, q_col, row_scale_inv_out, col_scale_inv_out, \
                  amax_out, r, s
    if (row_fmt == kE4M3) {
        if (dtype == kBF16) return launch_hybrid_t<kE4M3, kBF16>(FP8Q_ARGS);
        return launch_hybrid_t<kE4M3, kF32>(FP8Q_ARGS);
    }
    if (dtype == kBF16) return launch_hybrid_t<kE5M2, kBF16>(FP8Q_ARGS);
    return launch_hybrid_t<kE5M2, kF32>(FP8Q_ARGS);
#undef FP8Q_ARGS
}

// Block quantization runs at most 1024 blocks, each looping over tiles: its
// per-tile work ends in block-wide reductions and scattered scale stores, and
// a block's next tile overlaps them.  Measured on the MI355X (bf16, with
// columnwise codes): 1x128 blocks of 4096x7168 take 29.9 us against 31.6 us
// with one tile per block, 128x128 blocks of 7168x4096 26.1 against 26.6 us;
// the per-tensor rowwise/columnwise and MXFP8 casts, with no block-wide step
// per tile, are faster with one tile per block (55.0 vs 56.3 us and 63.2 vs
// 64.8 us at 8192x8192) and keep it.  Loading the next tile's input before
// working on the current one did not pay: 1x128 blocks 30.7 against 28.5 us,
// 128x128 blocks 25.7 against 24.8 us (24.8 with 512 blocks).
constexpr int kBlockQuantGrid = 1024;

template <int F, int DT>
static hipError_t launch_block_t(const void *x, int64_t rows, int64_t cols, int block_rows, uint8_t *q_row,
                                 float *s_row, uint8_t *q_col, float *s_col, hipStream_t s)
{
    const int grid = min(tile_grid(rows, cols), kBlockQuantGrid);
    const ScaleSrc none{nullptr, nullptr, 0};
    if (block_rows == 128)
        tile_kernel<F, DT, kTileBlock128, false><<<grid, kThreads, 0, s>>>(x, rows, cols, none, q_row, q_col, s_row,
                                                                          s_col, nullptr, nullptr, nullptr, none,
                                                                          nullptr, Finish{});
    else
        tile_kernel<F, DT, kTileBlock1x128, false><<<grid, kThreads, 0, s>>>(x, rows, cols, none, q_row, q_col,
                                                                            s_row, s_col, nullptr, nullptr, nullptr,
                                                                            none, nullptr, Finish{});
    return hipGetLastError();
}

template <int F, int DT>
static hipError_t launch_mx_t(const void *x, int64_t rows, int64_t cols, uint8_t *q_row, uint8_t *s_row,
                              uint8_t *q_col, uint8_t *s_col, hipStream_t s)
{
    const ScaleSrc none{nullptr, nullptr, 0};
    tile_kernel<F, DT, kTileMX, false><<<tile_grid(rows, cols), kThreads, 0, s>>>(
        x, rows, cols, none, q_row, q_col, s_row, s_col, nullptr, nullptr, nullptr, none, nullptr, Finish{});
    return hipGetLastError();
}

hipError_t launch_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t *q_row, uint8_t *s_row,
                     uint8_t *q_col, uint8_t *s_col, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    if (fmt == kE4M3) {
        if (dtype == kBF16) return launch_mx_t<kE4M3, kBF16>(x, rows, cols, q_row, s_row, q_col, s_col, s);
        return launch_mx_t<kE4M3, kF32>(x, rows, cols, q_row, s_row, q_col, s_col, s);
    }
    if (dtype == kBF16) return launch_mx_t<kE5M2, kBF16>(x, rows, cols, q_row, s_row, q_col, s_col, s);
    return launch_mx_t<kE5M2, kF32>(x, rows, cols, q_row, s_row, q_col, s_col, s);
}

// The buffers and the per-tensor scale source of one per-direction pass.
struct SubqArgs {
    const void *x;
    int64_t rows, cols;
    uint8_t *q_row;
    void *s_row; // block scales, or the one float a per-tensor direction reports its s in
    uint8_t *q_col;
    void *s_col;
    ScaleSrc pt; // the per-tensor direction's scale source
};

// One pass over x: the row codes by the recipe kMode in F, the column codes by
// the recipe kColMode in FC (block recipes, or per-tensor scaling in one of
// the two directions), from x or (kDeq) from the dequantized row codes;
// either copy may be absent (its code and scale pointers null).  A pass with
// MXFP8 or per-tensor codes runs one tile per block, the block-scaled ones
// loop over tiles (the measured faster forms).
template <int F, int FC, int DT, int kMode, int kColMode, bool kDeq>
static hipError_t launch_subq_m(const SubqArgs &a, hipStream_t s)
{
    constexpr bool kRowT = kMode == kTilePerTensor, kColT = kColMode == kTilePerTensor;
    const int grid = (kMode == kTileMX || kColMode == kTileMX || kRowT || kColT)
                         ? tile_grid(a.rows, a.cols)
                         : min(tile_grid(a.rows, a.cols), kBlockQuantGrid);
    const ScaleSrc none{nullptr, nullptr, 0};
    tile_kernel<F, DT, kMode, false, FC, kColMode, kDeq><<<grid, kThreads, 0, s>>>(
        a.x, a.rows, a.cols, kRowT ? a.pt : none, a.q_row, a.q_col, kRowT ? nullptr : a.s_row,
        kColT ? nullptr : a.s_col, kRowT ? reinterpret_cast<float *>(a.s_row) : nullptr, nullptr, nullptr,
        kColT ? a.pt : none, kColT ? reinterpret_cast<float *>(a.s_col) : nullptr, Finish{});
    return hipGetLastError();
}

template <int F, int FC, int DT, int kMode, bool kDeq>
static hipError_t launch_subq_c(int col_recipe, const SubqArgs &a, hipStream_t s)
{
    switch (col_recipe) {
    case kSubqBlock128: return launch_subq_m<F, FC, DT, kMode, kTileBlock128, kDeq>(a, s);
    case kSubqBlock1x128: return launch_subq_m<F, FC, DT, kMode, kTileBlock1x128, kDeq>(a, s);
    case kSubqMX: return launch_subq_m<F, FC, DT, kMode, kTileMX, kDeq>(a, s);
    case kSubqTensor:
        // (two per-tensor directions are the per-tensor hybrid's, not this pass's)
        if constexpr (kMode != kTilePerTensor) return launch_subq_m<F, FC, DT, kMode, kTilePerTensor, kDeq>(a, s);
        break;
    }
    return hipErrorInvalidValue;
}

template <int F, int FC, int DT, bool kDeq>
static hipError_t launch_subq_r(int row_recipe, int col_recipe, const SubqArgs &a, hipStream_t s)
{
    switch (row_recipe) {
    case kSubqBlock128: return launch_subq_c<F, FC, DT, kTileBlock128, kDeq>(col_recipe, a, s);
    case kSubqBlock1x128: return launch_subq_c<F, FC, DT, kTileBlock1x128, kDeq>(col_recipe, a, s);
    case kSubqMX: return launch_subq_c<F, FC, DT, kTileMX, kDeq>(col_recipe, a, s);
    case kSubqTensor: return launch_subq_c<F, FC, DT, kTilePerTensor, kDeq>(col_recipe, a, s);
    }
    return hipErrorInvalidValue;
}

template <int F, int FC>
static hipError_t launch_subq_d(int dtype, bool deq, int row_recipe, int col_recipe, const SubqArgs &a,
                                hipStream_t s)
{
    if (deq) {
        if (dtype == kBF16) return launch_subq_r<F, FC, kBF16, true>(row_recipe, col_recipe, a, s);
        return launch_subq_r<F, FC, kF32, true>(row_recipe, col_recipe, a, s);
    }
    if (dtype == kBF16) return launch_subq_r<F, FC, kBF16, false>(row_recipe, col_recipe, a, s);
    return launch_subq_r<F, FC, kF32, false>(row_recipe, col_recipe, a, s);
}

hipError_t launch_hybrid_blockwise(const void *x, int dtype, int64_t rows, int64_t cols, int row_recipe, int row_fmt,
                                   uint8_t *q_row, void *s_row, int col_recipe, int col_fmt, uint8_t *q_col,
                                   void *s_col, bool col_from_rows, ScaleSrc pt, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    // one direction alone: the single-format kernel of its recipe (the
    // dequantized source still forms the row codes, unstored); a per-tensor
    // direction alone pairs with an unstored block copy of the other
    const bool deq = col_from_rows && q_col;
    if (!q_col) {
        col_recipe = row_recipe == kSubqTensor ? kSubqBlock128 : row_recipe;
        col_fmt = row_fmt;
    }
    if (!q_row && !deq) {
        row_recipe = col_recipe == kSubqTensor ? kSubqBlock128 : col_recipe;
        row_fmt = col_fmt;
    }
    const SubqArgs a{x, rows, cols, q_row, s_row, q_col, s_col, pt};
    if (row_fmt == kE4M3)
        return col_fmt == kE4M3 ? launch_subq_d<kE4M3, kE4M3>(dtype, deq, row_recipe, col_recipe, a, s)
                                : launch_subq_d<kE4M3, kE5M2>(dtype, deq, row_recipe, col_recipe, a, s);
    return col_fmt == kE4M3 ? launch_subq_d<kE5M2, kE4M3>(dtype, deq, row_recipe, col_recipe, a, s)
                            : launch_subq_d<kE5M2, kE5M2>(dtype, deq, row_recipe, col_recipe, a, s);
}

hipError_t launch_block(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, int block_rows, uint8_t *q_row,
                        float *s_row, uint8_t *q_col, float *s_col, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    if (fmt == kE4M3) {
        if (dtype == kBF16) return launch_block_t<kE4M3, kBF16>(x, rows, cols, block_rows, q_row, s_row, q_col, s_col, s);
        return launch_block_t<kE4M3, kF32>(x, rows, cols, block_rows, q_row, s_row, q_col, s_col, s);
    }
    if (dtype == kBF16) return launch_block_t<kE5M2, kBF16>(x, rows, cols, block_rows, q_row, s_row, q_col, s_col, s);
    return launch_block_t<kE5M2, kF32>(x, rows, cols, block_rows, q_row, s_row, q_col, s_col, s);
}

} // namespace fp8q
