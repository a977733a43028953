// fp8q_device.h -- device-side building blocks of the gfx950 FP8 kernels:
// the scaled saturating cast, magnitude-bit maxima, wavefront and block
// reductions, and the scale arithmetic.
//
// Pages cited (title, section): "Megatron FP8" (sections 1-28).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// FP8_MAX per format ("Megatron FP8", section 2: 448 for E4M3FN, 57344 for
// E5M2) and the code of +FP8_MAX.
template <int F> struct Fmt;
template <> struct Fmt<kE4M3> {
    static constexpr float kMax = 448.0f;
    static constexpr uint32_t kMaxCode = 0x7E;
};
template <> struct Fmt<kE5M2> {
    static constexpr float kMax = 57344.0f;
    static constexpr uint32_t kMaxCode = 0x7B;
};

// The amax floor of current scaling ("Megatron FP8", section 4: amax is
// clamped below at 1e-12 before the division).
constexpr float kAmaxFloor = 1e-12f;
constexpr uint32_t kCanonicalNaN = 0x7FC00000u;
constexpr uint32_t kInfBits = 0x7F800000u;

// ---------------------------------------------------------------- cast ----
// Two scaled values -> two codes in the low (kHi = false) or high half of a
// dword.  The hardware converter rounds to nearest even but does not
// saturate, so the value is first clamped to [-FP8_MAX, FP8_MAX] with med3.
// med3 turns NaN into -FP8_MAX; encode4s / encode1 repair NaN lanes.
template <int F, bool kHi>
__device__ __forceinline__ int cvt2(float a, float b, int old)
{
    const float ca = __builtin_amdgcn_fmed3f(a, -Fmt<F>::kMax, Fmt<F>::kMax);
    const float cb = __builtin_amdgcn_fmed3f(b, -Fmt<F>::kMax, Fmt<F>::kMax);
    if constexpr (F == kE4M3)
        return __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, old, kHi);
    else
        return __builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, old, kHi);
}

// Code byte of a NaN product x*scale: 0x7F with the sign bit
// sign(x) XOR sign(scale).
__device__ __forceinline__ uint32_t nan_code(float x, float scale)
{
    return 0x7Fu | (((__float_as_uint(x) ^ __float_as_uint(scale)) >> 24) & 0x80u);
}

// Four elements x[k] times their scales s[k] -> one dword of four codes
// (byte k = code of x[k] * s[k]).  kRepair = false is for callers that have
// shown no product can be NaN (no NaN input, every scale finite and nonzero):
// it skips the NaN test.
template <int F, bool kRepair = true>
__device__ __forceinline__ uint32_t encode4s(float x0, float x1, float x2, float x3, float s0, float s1, float s2,
                                             float s3)
{
    const float y0 = x0 * s0, y1 = x1 * s1, y2 = x2 * s2, y3 = x3 * s3;
    int r = cvt2<F, false>(y0, y1, 0);
    r = cvt2<F, true>(y2, y3, r);
    uint32_t c = (uint32_t)r;
    if constexpr (!kRepair) return c;
    // NaN products are rare: one compare per element, a branch per dword.
    const bool any_nan = (y0 != y0) | (y1 != y1) | (y2 != y2) | (y3 != y3);
    if (__builtin_expect(any_nan, 0)) {
        if (y0 != y0) c = (c & 0xFFFFFF00u) | nan_code(x0, s0);
        if (y1 != y1) c = (c & 0xFFFF00FFu) | (nan_code(x1, s1) << 8);
        if (y2 != y2) c = (c & 0xFF00FFFFu) | (nan_code(x2, s2) << 16);
        if (y3 != y3) c = (c & 0x00FFFFFFu) | (nan_code(x3, s3) << 24);
    }
    return c;
}

// Four elements with one scale.
template <int F, bool kRepair = true>
__device__ __forceinline__ uint32_t encode4(float x0, float x1, float x2, float x3, float scale)
{
    return encode4s<F, kRepair>(x0, x1, x2, x3, scale, scale, scale, scale);
}

// A scale with which no finite input gives a NaN product.
__device__ __forceinline__ bool finite_nonzero(float s) { return fabsf(s) < __builtin_inff() && s != 0.0f; }

// One element -> its code byte.
template <int F>
__device__ __forceinline__ uint32_t encode1(float x, float scale)
{
    const float y = x * scale;
    const uint32_t c = (uint32_t)cvt2<F, false>(y, y, 0) & 0xFFu;
    return (y != y) ? nan_code(x, scale) : c;
}

// ------------------------------------------------------ streaming access --
// Every element of a streamed tensor is touched once per pass, so the
// element kernels load and store with the non-temporal hint: the lines are
// not kept in L2 or the last-level cache, which leaves those to the data that
// is re-used.  Measured on the MI355X over 128 MiB inputs: a read-only pass
// moves 6.7 TB/s with the hint against 6.2 TB/s without, and a 2-byte read /
// 1-byte write pass (the bf16 cast) 8% faster with both hints.  The one
// exception is the tail of the amax pass, which the cast of current scaling
// reads again at once (amax_kernel keeps it in the caches).
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const void *p)
{
    const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st_stream(void *p, uint4 v)
{
    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v *>(p));
}

__device__ __forceinline__ uint32_t ld_stream_u32(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}

// bf16 pair in a dword -> two exact floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------- magnitude max ----
// The amax of a tensor is the maximum of |x| over magnitude bit patterns:
// for non-negative IEEE values the unsigned order of the bits is the numeric
// order, and every NaN pattern lies above +Inf, so the integer maximum is
// exact, independent of order, and detects NaN.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t w)
{
    u16x2 v;
    __builtin_memcpy(&v, &w, 4);
    return v;
}

// running max of the two bf16 magnitudes held in w (packed 16-bit max)
__device__ __forceinline__ u16x2 bf16_absmax2(u16x2 acc, uint32_t w)
{
    return __builtin_elementwise_max(acc, as_u16x2(w & 0x7FFF7FFFu));
}

// packed bf16 magnitude max -> fp32 magnitude bits
__device__ __forceinline__ uint32_t bf16_absmax_to_f32bits(u16x2 acc)
{
    const uint32_t m = acc.x > acc.y ? acc.x : acc.y;
    return m << 16;
}

__device__ __forceinline__ uint32_t f32_absbits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// A magnitude maximum in fp32 bits -> the amax value's bits (NaN -> canonical).
__device__ __forceinline__ uint32_t canonical_amax_bits(uint32_t m) { return m > kInfBits ? kCanonicalNaN : m; }

// ---------------------------------------------------------- reductions ----
// Wavefront (64 lanes) max of an unsigned value with DPP row shifts and row
// broadcasts; the result is valid in lane 63 and returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    // row_shr:1,2,4,8 give each lane 15 of every 16-lane row the row max
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
    // row_bcast:15 (rows 1 and 3) and row_bcast:31 (rows 2 and 3)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Max with the value of lane ^ 16 or lane ^ 32, through gfx950's lane-swap
// instructions (vector ALU, no LDS round trip): with both operands the same
// register, v_permlane16_swap leaves each lane its own value in one result
// and its lane ^ 16 partner's in the other (odd and even 16-lane rows
// exchanged), v_permlane32_swap likewise for the two 32-lane halves; the max
// of the two results is the pair's max in every lane (checked lane by lane on
// the MI355X).
__device__ __forceinline__ uint32_t max_xor16(uint32_t m)
{
    const auto p = __builtin_amdgcn_permlane16_swap(m, m, false, false);
    return max((uint32_t)p[0], (uint32_t)p[1]);
}
__device__ __forceinline__ uint32_t max_xor32(uint32_t m)
{
    const auto p = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return max((uint32_t)p[0], (uint32_t)p[1]);
}

// Block max (blockDim.x = kThreads, a multiple of 64); every thread gets the
// result.  `lds` must hold kThreads/64 words.
template <int kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *lds)
{
    constexpr int kWaves = kThreads / 64;
    v = wave_max_u32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    uint32_t r = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = max(r, lds[w]);
    __syncthreads();
    return r;
}

// ------------------------------------------------- grid-wide amax partials --
// A producing block publishes its canonical magnitude max (below 2^31) to its
// slot as tag << 32 | bits, the tag being the call's (nonzero, new for every
// call on the slot).  The store is a 64-bit agent-scope atomic, visible to
// the agent-scope loads of a finishing block running on another XCD while
// the launch still runs.
__device__ __forceinline__ void publish_partial(unsigned long long *slot, uint32_t tag, uint32_t canonical_bits)
{
    __hip_atomic_store(slot, ((unsigned long long)tag << 32) | canonical_bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// The finishing block of a launch (its last block, after the producing
// blocks): every lane polls its slots of pub[0, nparts) with agent-scope
// loads, sleeping briefly between rounds, until the whole block has seen all
// nparts slots carry the call's tag; then every lane gets the max of their
// values, and the slots are put back to zero, so that a launch replayed from
// a captured graph (same tag) waits for its own partials again.  It waits
// only for the other blocks of its launch, which never wait, so the wait ends
// once they have run; it is bounded all the same, by `rounds` polling rounds,
// after which the result is the canonical NaN (a partial that arrives later
// carries a tag no later call accepts).  This replaces a second, one-block
// kernel whose launch would follow the producers' end.  NT lanes, nparts <=
// kMax, kMax a multiple of NT.
template <int NT, int kMax>
__device__ __forceinline__ uint32_t collect_partials(unsigned long long *pub, int nparts, uint32_t tag,
                                                     uint32_t rounds)
{
    __shared__ uint32_t red[NT / 64];
    constexpr int kPer = kMax / NT;
    static_assert(kPer * NT == kMax && kPer <= 32, "slots per lane");
    uint32_t m = 0;
    uint32_t left = 0; // bit u: slot threadIdx.x + u * NT not seen yet
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        if ((int)threadIdx.x + u * NT < nparts) left |= 1u << u;
    bool expired = true;
    for (uint32_t round = 0; round < rounds; ++round) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (left & (1u << u)) {
                const unsigned long long v =
                    __hip_atomic_load(&pub[threadIdx.x + u * NT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((uint32_t)(v >> 32) == tag) {
                    m = max(m, (uint32_t)v);
                    left &= ~(1u << u);
                }
            }
        }
        if (__syncthreads_and(left == 0)) { // block-uniform
            expired = false;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        if ((int)threadIdx.x + u * NT < nparts)
            __hip_atomic_store(&pub[threadIdx.x + u * NT], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    m = block_max_u32<NT>(m, red);
    return expired ? kCanonicalNaN : m;
}

// ------------------------------------------------------ scale arithmetic --
// Current scaling ("Megatron FP8", sections 4 and 10):
//   s = fl32(max(amax, 1e-12) / FP8_MAX) * 2^margin   (dequant multiplier)
//   scale = fl32(1 / s)                                (quant multiplier)
// The divisions are IEEE correctly rounded (the default for HIP float
// division); a NaN amax propagates.
struct Scales {
    float s;     // scale_inv: value = code value * s
    float scale; // quantization multiplier
};

__device__ __forceinline__ Scales current_scales(float amax, float fmax, int margin)
{
    const float ac = (amax != amax) ? amax : (amax > kAmaxFloor ? amax : kAmaxFloor);
    const float s = ldexpf(ac / fmax, margin);
    return Scales{s, 1.0f / s};
}

__device__ __forceinline__ Scales given_scales(float s) { return Scales{s, 1.0f / s}; }

} // namespace fp8q
