// gemm.hip -- scaled FP8 GEMM on gfx950 matrix cores.
//
// C[M][N] = (A*sA)(B*sB)^T with A [M][K], B [N][K] FP8 codes (K-contiguous),
// fp32 accumulation in v_mfma_f32_16x16x128_f8f6f4 and a bf16 output.
//   per-tensor: C = bf16(fl32(fl32(sA*sB) * acc))                 ("Megatron FP8",
//               section 6: fp32 accumulate, bf16 out; section 27: one downcast
//               of the finished dot product)
//   block:      each 128-wide K slice is its own MFMA partial, promoted into the
//               fp32 accumulator with the 1x128 scale of A's row and the
//               128x128 scale of B's block: acc += (sA[m,kb]*sB[n/128,kb]) * part
// and, optionally, amax_out = max |C| over the emitted bf16 values.
//
// Tiling: a 128x128 output tile per block of 256 lanes (four waves in 2x2, each
// 64x64 = 4x4 MFMA tiles of 16x16), K in steps of 128 bytes.  Both operand
// tiles (16 KiB each) are staged in LDS, double-buffered, with the 16-byte
// chunks of each 128-byte row XOR-swizzled by the row index so that the
// fragment reads of a wave spread over the banks.  A and B fragments are read
// with the same lane -> K mapping, so the MFMA's internal K order does not
// affect the dot product.  Blocks are remapped so that the tiles resident on
// one XCD (blocks are dealt round-robin to the 8 XCDs) form contiguous groups
// of rows and columns of C, which keeps their operand panels in that XCD's L2.
#include "fp8q_device.h"
#include "fp8q_launch.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kGemmThreads = 256;
constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kXcds = 8;
constexpr int kGroupM = 8; // tile rows per L2 group

template <int FA, int FB>
__device__ __forceinline__ v4f mfma16x16x128(const v8i &a, const v8i &b, const v4f &c)
{
    // cbsz / blgp select the operand formats (0 = E4M3, 1 = E5M2); zero
    // scale operands select the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// byte offset of 16-byte chunk c of row r in a [128][128] LDS tile
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ void tile_of_block(int bid, int tilesM, int tilesN, int &tm, int &tn)
{
    const int ntiles = tilesM * tilesN;
    int t = bid;
    if (ntiles % kXcds == 0) t = (bid % kXcds) * (ntiles / kXcds) + bid / kXcds;
    const int per_group = kGroupM * tilesN;
    const int group = t / per_group;
    const int first_m = group * kGroupM;
    const int gsize = min(tilesM - first_m, kGroupM);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

template <int FA, int FB, bool kBlock, bool kAmax>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_kernel(const uint8_t *__restrict__ A,
                                                               const uint8_t *__restrict__ B,
                                                               const float *__restrict__ sA,
                                                               const float *__restrict__ sB, int M, int N, int K,
                                                               __bf16 *__restrict__ C, GridScratch *gs,
                                                               uint32_t *__restrict__ amax_out)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kBM * kBK];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kBN * kBK];
    __shared__ __attribute__((aligned(16))) float lds_sa[kBlock ? 2 : 1][kBlock ? kBM : 1];
    __shared__ uint32_t red[kGemmThreads / 64];

    int tm, tn;
    tile_of_block(blockIdx.x, M / kBM, N / kBN, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int nk = K / kBK;
    const int kblocks = K / 128;

    // global -> LDS staging: lane loads rows ld_row + 32u, chunk ld_chunk
    const int ld_row = tid >> 3, ld_chunk = tid & 7;
    const uint8_t *Ag = A + (m0 + ld_row) * (int64_t)K + ld_chunk * 16;
    const uint8_t *Bg = B + (n0 + ld_row) * (int64_t)K + ld_chunk * 16;
    uint4 ra[4], rb[4];
    float rsa = 0.f;

    auto gload = [&](int kt) {
        const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ra[u] = *reinterpret_cast<const uint4 *>(Ag + (int64_t)(32 * u) * K + k0);
            rb[u] = *reinterpret_cast<const uint4 *>(Bg + (int64_t)(32 * u) * K + k0);
        }
        if constexpr (kBlock) {
            if (tid < kBM) rsa = sA[(m0 + tid) * kblocks + kt];
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = ld_row + 32 * u;
            *reinterpret_cast<uint4 *>(&lds_a[buf][swz(r, ld_chunk)]) = ra[u];
            *reinterpret_cast<uint4 *>(&lds_b[buf][swz(r, ld_chunk)]) = rb[u];
        }
        if constexpr (kBlock) {
            if (tid < kBM) lds_sa[buf][tid] = rsa;
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();

    const int fr = lane & 15, fg = lane >> 4; // fragment row within 16, K group
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);

        v8i a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + 16 * i + fr;
            const uint4 lo = *reinterpret_cast<const uint4 *>(&lds_a[cur][swz(r, 2 * fg)]);
            const uint4 hi = *reinterpret_cast<const uint4 *>(&lds_a[cur][swz(r, 2 * fg + 1)]);
            a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn * 64 + 16 * j + fr;
            const uint4 lo = *reinterpret_cast<const uint4 *>(&lds_b[cur][swz(r, 2 * fg)]);
            const uint4 hi = *reinterpret_cast<const uint4 *>(&lds_b[cur][swz(r, 2 * fg + 1)]);
            b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }

        if constexpr (kBlock) {
            // promote this K block's partials with the two block scales
            const float sb = sB[(n0 / 128) * kblocks + kt];
            v4f wsc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 sa = *reinterpret_cast<const float4 *>(&lds_sa[cur][wm * 64 + 16 * i + 4 * fg]);
                wsc[i] = v4f{sa.x * sb, sa.y * sb, sa.z * sb, sa.w * sb};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f part = mfma16x16x128<FA, FB>(a[i], b[j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(part[e], wsc[i][e], acc[i][j][e]);
                }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x128<FA, FB>(a[i], b[j], acc[i][j]);
        }

        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds rows 4*fg + e (e = 0..3) of column fr of each 16x16 tile
    const float alpha = kBlock ? 1.0f : (*sA) * (*sB);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 64 + 16 * j + fr;
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const f32x2 v = kBlock ? f32x2{acc[i][j][e], acc[i][j][e + 1]}
                                       : f32x2{acc[i][j][e] * alpha, acc[i][j][e + 1] * alpha};
                const bf16x2 h = __builtin_convertvector(v, bf16x2);
                const int64_t row = m0 + wm * 64 + 16 * i + 4 * fg + e;
                C[row * N + col] = h[0];
                C[(row + 1) * N + col] = h[1];
                if constexpr (kAmax) {
                    const uint32_t bits = __builtin_bit_cast(uint32_t, h);
                    m = max(m, (bits & 0x7FFFu) << 16);
                    m = max(m, (bits >> 16 & 0x7FFFu) << 16);
                }
            }
        }
    if constexpr (kAmax) {
        // last-block finish, as in the quantization kernels
        m = block_max_u32<kGemmThreads>(m, red);
        if (tid == 0) {
            atomicMax(&gs->max_bits, canonical_amax_bits(m));
            __threadfence();
            if (atomicAdd(&gs->ticket, 1u) == gridDim.x - 1) {
                __threadfence();
                const uint32_t v = atomicExch(&gs->max_bits, 0u);
                atomicExch(&gs->ticket, 0u);
                *amax_out = v;
            }
        }
    }
}

template <int FA, int FB>
static hipError_t launch_gemm_t(const uint8_t *A, const float *sA, const uint8_t *B, const float *sB, int64_t M,
                                int64_t N, int64_t K, int mode, void *C, float *amax_out, GridScratch *gs,
                                hipStream_t s)
{
    const int grid = (int)((M / kBM) * (N / kBN));
    __bf16 *c = reinterpret_cast<__bf16 *>(C);
    uint32_t *am = reinterpret_cast<uint32_t *>(amax_out);
    const int m = (int)M, n = (int)N, k = (int)K;
    if (mode == 0) {
        if (am)
            gemm_kernel<FA, FB, false, true><<<grid, kGemmThreads, 0, s>>>(A, B, sA, sB, m, n, k, c, gs, am);
        else
            gemm_kernel<FA, FB, false, false><<<grid, kGemmThreads, 0, s>>>(A, B, sA, sB, m, n, k, c, gs, am);
    } else {
        if (am)
            gemm_kernel<FA, FB, true, true><<<grid, kGemmThreads, 0, s>>>(A, B, sA, sB, m, n, k, c, gs, am);
        else
            gemm_kernel<FA, FB, true, false><<<grid, kGemmThreads, 0, s>>>(A, B, sA, sB, m, n, k, c, gs, am);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t *A, int fa, const float *sA, const uint8_t *B, int fb, const float *sB, int64_t M,
                       int64_t N, int64_t K, int mode, void *C, float *amax_out, GridScratch *gs, hipStream_t s)
{
    if (fa == kE4M3 && fb == kE4M3)
        return launch_gemm_t<kE4M3, kE4M3>(A, sA, B, sB, M, N, K, mode, C, amax_out, gs, s);
    if (fa == kE5M2 && fb == kE4M3)
        return launch_gemm_t<kE5M2, kE4M3>(A, sA, B, sB, M, N, K, mode, C, amax_out, gs, s);
    if (fa == kE4M3 && fb == kE5M2)
        return launch_gemm_t<kE4M3, kE5M2>(A, sA, B, sB, M, N, K, mode, C, amax_out, gs, s);
    return launch_gemm_t<kE5M2, kE5M2>(A, sA, B, sB, M, N, K, mode, C, amax_out, gs, s);
}

} // namespace fp8q
