// gemm_kernels.h -- scaled FP8 GEMM kernels for gfx950 matrix cores, included
// by one translation unit per operand-format pair (gemm_<fa>_<fb>.hip), which
// lets the instantiations compile in parallel.
//
// C[M][N] = epi((A*sA)(B*sB)^T) with A [M][K], B [N][K] FP8 codes
// (K-contiguous) and fp32 accumulation on the f8f6f4 matrix instructions
// ("Megatron FP8", section 6: FP8 operands, fp32 accumulation, bf16 output for
// fprop / dgrad and fp32 output for wgrad; section 27: products promoted to
// fp32 and summed, one downcast of the finished dot product).
//   per-tensor: v = fl32(fl32(sA*sB) * acc)
//   block:      each 128-wide K slice is its own MFMA partial, promoted into
//               the fp32 accumulator with the slice's two block scales:
//               acc = fma(part, fl32(sA[m,kb]*sB[.,kb]), acc), v = acc, with
//               B's scale per 128x128 block or per row (1x128)
//   MXFP8:      the E8M0 block scales are applied by the matrix instruction
// The epilogue writes bf16 (RNE), fp32 or FP8 codes of act(v + bias), and
// optionally the per-block magnitude max of what it emits (folded into
// amax_out by the finish kernel).  Results go through the LDS stages (free
// once the K loop is done) and leave as whole row pieces.
//
// Two kernels, both with 256x256 block tiles and operand tiles moved from
// global memory straight into LDS by buffer loads (no register staging),
// 16-byte chunks XOR-swizzled by row so that fragment reads spread over the
// LDS banks:
//
//   gemm_pt_kernel (per-tensor and MXFP8): four waves of 128x128, each as 4x4
//   tiles of 32x32 (v_mfma_scale_f32_32x32x64_f8f6f4, 256 accumulators); K
//   moves in slices of 128 through two LDS stages.
//
//   gemm_bs_pp_kernel (block-scaled): eight waves of 64x128, each as 4x8
//   tiles of 16x16 (v_mfma_f32_16x16x128_f8f6f4), in two groups that take
//   turns at the matrix pipes; K moves in steps of 128 (one block-scale slice)
//   through two LDS stages, and each slice's partial is promoted on the
//   vector ALU.
//
// Operand order.  The MFMA is issued as (B fragment, A fragment), so its
// result is C^T: in a 16x16 tile lane (r = lane % 16, g = lane / 16) holds
// C[r][4g..4g+3], four consecutive columns of one row, stored as one 8-byte
// bf16 quad (32x32 tiles likewise, per group of four accumulators).  A and B
// fragments use the same lane -> K mapping, so the MFMA's internal K order does
// not affect the dot product.
//
// Blocks are dealt round-robin to the 8 XCDs; the tile index is remapped so
// that each XCD works on a compact group of output tiles (4 tile rows wide),
// whose operand panels then stay in that XCD's L2.
#ifndef FP8Q_GEMM_KERNELS_H
#define FP8Q_GEMM_KERNELS_H

#include "fp8q_device.h"
#include "fp8q_launch.h"
#include "gemm_pairs.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
constexpr int kBM = 256, kBK = 128;
constexpr int kXcds = 8;
constexpr int kGroupM = 4; // tile rows per L2 group
constexpr uint32_t kRawBufferWord3 = 0x00020000u;

template <int FX, int FY>
__device__ __forceinline__ v4f mfma16x16x128(const v8i &x, const v8i &y, const v4f &c)
{
    // cbsz / blgp give the formats of the two operands (0 = E4M3, 1 = E5M2);
    // zero scale operands select the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, FX, FY, 0, 0, 0, 0);
}

// Byte offset of 16-byte chunk c of row r in a [rows][128] LDS stage.  The LDS
// serves 256 bytes (64 banks) per cycle, i.e. two 128-byte rows; XOR-ing the
// chunk with bits 1..3 of the row gives the 16 rows read by 16 lanes of a
// fragment 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * kBK + ((c ^ ((r >> 1) & 7)) << 4); }

// Tile t of the grouped order: groups of kGroupM tile rows, walked column by
// column inside a group.
__device__ __forceinline__ void group_tile(int t, int tilesM, int tilesN, int &tm, int &tn)
{
    const int per_group = kGroupM * tilesN;
    const int group = t / per_group;
    const int first_m = group * kGroupM;
    const int gsize = min(tilesM - first_m, kGroupM);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Block bid of a grid of n blocks -> its index in the grouped order, dealt so
// that each XCD gets a contiguous run (blocks go to XCD bid mod 8).
__device__ __forceinline__ int xcd_order(int bid, int n) { return n % kXcds ? bid : (bid % kXcds) * (n / kXcds) + bid / kXcds; }

__device__ __forceinline__ void tile_of_block(int bid, int tilesM, int tilesN, int &tm, int &tn)
{
    group_tile(xcd_order(bid, tilesM * tilesN), tilesM, tilesN, tm, tn);
}

typedef __attribute__((address_space(3))) void lds_void;

// One operand fragment (16 rows x 128 K bytes): lane (r, g) reads logical
// chunks g and g + 4 of row r.  (Chunks 2g and 2g + 1 would be the same K
// bytes in another order, but then lanes r and r + 16 of one read hit the same
// banks: measured, that read pattern runs at 0.6x the speed with half of the
// LDS cycles lost to bank conflicts.)
__device__ __forceinline__ v8i read_frag(const uint8_t *lds, int r, int g)
{
    const uint4 lo = *reinterpret_cast<const uint4 *>(lds + swz(r, g));
    const uint4 hi = *reinterpret_cast<const uint4 *>(lds + swz(r, g + 4));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Output kinds of the epilogue: bf16 (round to nearest even), fp32, or FP8
// codes of either format (the fused epilogue of the next layer's cast).
enum OutKind { kOutBF16 = 0, kOutF32 = 1, kOutE4M3 = 2, kOutE5M2 = 3 };

// Fused epilogue ("Megatron FP8", section 6: bias and activation folded into
// the GEMM epilogue so the intermediate never round-trips through memory;
// section 4: the output cast with its own scale, its amax recorded for the
// next scaling decision):
//   y = act(v + bias[col]), act: none, ReLU (v < 0 -> 0, NaN kept) or GELU;
//   FP8 output: codes of fl32(y * fl32(1 / *out_si)).
enum Act { kActNone = 0, kActRelu = 1, kActGelu = 2 };

// GELU(x) = x Phi(x), Phi the standard normal CDF.  The tail
// Q = Phi(-|x|) = erfc(z)/2, z = |x|/sqrt 2, is evaluated as
//   Q = t 2^(P(t) - z^2 log2 e),  t = 1 / (1 + 0.4 z),
// with P a degree-8 polynomial fitted in log2 over 0 <= z <= 9.5 (gelu_fit.py
// holds the fit and prints these coefficients); Phi = 1 - Q for x >= 0, Q
// otherwise.  Evaluated in binary32 the result is within 2^-21.6 |x| of
// x Phi(x); one reciprocal and one exp2 per value (the library erfc costs
// about three times the instructions, and in this epilogue every instruction
// is paid with the matrix cores idle).  x = +inf gives +inf, -inf and NaN give
// NaN, as x Phi(x) does.
__device__ __forceinline__ float gelu_f32(float x)
{
    const float zl = fabsf(x) * 0.849321783f; // z sqrt(log2 e)
    const float t = __builtin_amdgcn_rcpf(fmaf(zl, 0.333021849f, 1.0f));
    float p = -0.297103107f;
    p = fmaf(p, t, 1.32235646f);
    p = fmaf(p, t, -2.11821508f);
    p = fmaf(p, t, 1.4100548f);
    p = fmaf(p, t, -0.616400838f);
    p = fmaf(p, t, 0.422621727f);
    p = fmaf(p, t, 0.579714179f);
    p = fmaf(p, t, 1.4447f);
    p = fmaf(p, t, -3.14772844f);
    const float q = t * __builtin_amdgcn_exp2f(fmaf(-zl, zl, p));
    return x * (x >= 0.0f ? 1.0f - q : q);
}

struct Epi {
    const float *bias;   // [N] or null
    int act;
    const float *out_si; // the output's dequant scale s (FP8 output only)
};

// Apply the epilogue to four consecutive outputs of one row of C (starting at
// column col) and return their bytes packed from the low end (bf16: 8, fp32:
// 16, FP8: 4), folding their magnitudes into m (canonicalised later): for bf16
// and fp32 outputs the emitted values, for FP8 outputs the values y before the
// cast.
template <int kOut, bool kAmax, bool kFuse>
__device__ __forceinline__ uint4 pack_out4(int64_t col, v4f v, uint32_t &m, const Epi &epi, float out_scale)
{
    if constexpr (kFuse) {
        // v is already rounded to binary32; the bias add rounds once more (no
        // fused multiply-add with the scale that formed v)
#pragma clang fp contract(off)
        if (epi.bias) v += *reinterpret_cast<const v4f *>(epi.bias + col);
        if (epi.act == kActRelu) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = v[e] < 0.0f ? 0.0f : v[e];
        } else if (epi.act == kActGelu) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_f32(v[e]);
        }
    }
    if constexpr (kOut == kOutF32) {
        if constexpr (kAmax) {
#pragma unroll
            for (int e = 0; e < 4; ++e) m = max(m, __float_as_uint(v[e]) & 0x7FFFFFFFu);
        }
        return __builtin_bit_cast(uint4, v);
    } else if constexpr (kOut == kOutBF16) {
        const uint2 bits = __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4));
        if constexpr (kAmax) {
            m = max(m, max((bits.x & 0x7FFFu) << 16, (bits.x >> 16 & 0x7FFFu) << 16));
            m = max(m, max((bits.y & 0x7FFFu) << 16, (bits.y >> 16 & 0x7FFFu) << 16));
        }
        return make_uint4(bits.x, bits.y, 0u, 0u);
    } else {
        constexpr int F = kOut == kOutE4M3 ? kE4M3 : kE5M2;
        if constexpr (kAmax) {
#pragma unroll
            for (int e = 0; e < 4; ++e) m = max(m, __float_as_uint(v[e]) & 0x7FFFFFFFu);
        }
        return make_uint4(encode4<F>(v[0], v[1], v[2], v[3], out_scale), 0u, 0u, 0u);
    }
}

template <int kOut> constexpr int out_bytes() { return kOut == kOutF32 ? 4 : kOut == kOutBF16 ? 2 : 1; }

// A wave's output tile staged through LDS (the operand stages, free once the K
// loop is done) and stored as whole row pieces.  The matrix-instruction
// layout leaves each lane four consecutive values of one row, so a direct
// store instruction would write 4 to 16 bytes into each of 16 or 32 rows;
// from LDS each store instruction writes 16 bytes per lane along rows of
// kCols * kB contiguous bytes.  Rows are kCols * kB bytes whose 16-byte chunks
// are XOR-swizzled by the row, so that both the quad writes and the row reads
// spread over the banks.  A pass holds kPassRows rows (the whole wave tile
// unless fp32 does not fit the wave's share of the stages).  The stores carry
// the non-temporal hint: C is not read again by the kernel, and measured on
// the MI355X every GEMM ran the same or up to 2% faster with it (the
// weight-gradient GEMM with fp32 output 280.1 -> 274.5 us, 8192^3 per-tensor
// 374.7 -> 371.0 us, same box).
template <int kCols, int kB, int kRows, int kBudget> struct EpiStage {
    static constexpr int kPitch = kCols * kB, kNC = kPitch / 16, kRowsPerStore = 64 / kNC;
    static constexpr int kPassRows = kRows * kPitch <= kBudget ? kRows : kBudget / kPitch;
    static constexpr int kPasses = kRows / kPassRows;
    __device__ static __forceinline__ int addr(int r, int c) { return r * kPitch + ((c ^ (r & (kNC - 1))) << 4); }
    // packed bytes of quad h (columns 4h .. 4h + 3) of row r
    __device__ static __forceinline__ void put(uint8_t *ep, int r, int h, uint4 bits)
    {
        const int o = 4 * h * kB;
        uint8_t *p = ep + addr(r, o >> 4) + (o & 15);
        if constexpr (kB == 4) *reinterpret_cast<uint4 *>(p) = bits;
        else if constexpr (kB == 2) *reinterpret_cast<uint2 *>(p) = make_uint2(bits.x, bits.y);
        else *reinterpret_cast<uint32_t *>(p) = bits.x;
    }
    // kPassRows rows to C [.][N] (elements of kB bytes), from row0, col0
    __device__ static __forceinline__ void store(const uint8_t *ep, void *C, int64_t N, int64_t row0, int64_t col0,
                                                 int lane)
    {
        const int c = lane % kNC, rr = lane / kNC;
        uint8_t *Cb = reinterpret_cast<uint8_t *>(C);
#pragma unroll 4
        for (int s = 0; s < kPassRows / kRowsPerStore; ++s) {
            const int r = s * kRowsPerStore + rr;
            const uint4 v = *reinterpret_cast<const uint4 *>(ep + addr(r, c));
            st_stream(Cb + ((row0 + r) * N + col0) * kB + 16 * c, v);
        }
    }
};

// ---------------------------------------------------------------------------
// Per-tensor kernel.  256x256 block tile, 2x2 waves of 128x128 as 4x4 tiles
// of v_mfma_f32_32x32x64_f8f6f4 (256 fp32 accumulators per lane).  K moves in
// slices of 128 through two LDS stages of 64 KiB; every direct load moves 8
// rows x 128 bytes (whole 128-byte rows fetch about 1.6x faster from L2 than
// 64-byte half rows).  A slice is two half steps of 64 K, each 16 MFMAs per
// wave, and the one barrier per slice sits between them:
//   half 0: MFMAs on the slice's first-half fragments while the second-half
//           fragments are read from LDS;
//   sync:   wait for this lane's loads of the next slice and the LDS reads,
//           then barrier: the next slice is in LDS and nobody reads this
//           slice's stage any more;
//   half 1: the loads of the slice after next go into this stage, while the
//           MFMAs run on the second-half fragments and the next slice's
//           first-half fragments are read.
// So LDS reads always overlap MFMAs, and the loads have a whole slice of
// MFMAs to land.
constexpr int kPTStageBytes = 2 * kBM * kBK;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8).  Issued through the builtin rather than inline asm so
// that the compiler's own wait insertion knows what has been waited for.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 0xF) | (7 << 4) | ((lgkm & 0xF) << 8) | ((vm >> 4) << 14); }

typedef float v16f __attribute__((ext_vector_type(16)));

template <int FX, int FY>
__device__ __forceinline__ v16f mfma32x32x64(const v8i &x, const v8i &y, const v16f &c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, FX, FY, 0, 0, 0, 0);
}

// 32 rows x 64 K bytes of half step h: lane (r = lane % 32, g = lane / 32)
// reads logical chunks 4h + 2g and 4h + 2g + 1 of row r (same swizzle as above)
__device__ __forceinline__ v8i read_frag32(const uint8_t *lds, int r, int g, int h)
{
    const uint4 lo = *reinterpret_cast<const uint4 *>(lds + swz(r, 4 * h + 2 * g));
    const uint4 hi = *reinterpret_cast<const uint4 *>(lds + swz(r, 4 * h + 2 * g + 1));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// MXFP8 layout of the same 32 rows x 64 K bytes.  The scaled instruction's
// K order puts bytes 0..15 of lane (r, g) at K 16g .. 16g+15 of the half step
// and bytes 16..31 at K 32 + 16g .. 32 + 16g + 15, and takes the scale of K
// block b (32 elements) of row r from lane r + 32b (measured on the MI355X with
// unit codes and one scaled lane at a time).  So lane (r, g) reads logical
// chunks 4h + g and 4h + 2 + g, and supplies the scale of block 2h + g.
__device__ __forceinline__ v8i read_frag32_mx(const uint8_t *lds, int r, int g, int h)
{
    const uint4 lo = *reinterpret_cast<const uint4 *>(lds + swz(r, 4 * h + g));
    const uint4 hi = *reinterpret_cast<const uint4 *>(lds + swz(r, 4 * h + 2 + g));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// The two stages are distinct LDS objects addressed with compile-time stage
// numbers (the slice loop is unrolled by two), so the compiler can tell a
// read of one stage from the direct loads landing in the other.
// With kMX (MXFP8), sA and sB point to E8M0 scale bytes, [M][K/32] and
// [N][K/32]: every 32-element K block of a row carries a power of two that the
// matrix instruction applies itself (v_mfma_scale_f32_32x32x64_f8f6f4 takes one
// scale byte per lane, for the 32 K bytes that lane holds).  The scales come
// in groups of four slices: 16 bytes of every A and B row, loaded straight
// into LDS ([row][4 dwords], two groups in flight) by loads in which four
// lanes cover one row's 16 bytes, so each load touches 16 rows instead of 64
// (a load per slice of one scale dword per row, 64 rows apart in memory, kept
// the address unit busy and the slice's wait long).
// kBN = 256: a 256x256 tile per block (grid block b -> grouped tile
// xcd_order(b, n_main)); kBN = 128: half a tile, wave tiles 128x64 (grid
// block b -> half b & 1 of grouped tile tile_base + b / 2), for a last wave of
// tiles that is at most half full.  Each block's amax partial is folded into
// part[b % kParts] (an atomic max; the finish kernel reads and clears it).
template <int FA, int FB, bool kAmax, int kOut, bool kFuse, bool kMX, int kBN>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_pt_kernel(const uint8_t *__restrict__ A,
                                                                  const uint8_t *__restrict__ B,
                                                                  const float *__restrict__ sA,
                                                                  const float *__restrict__ sB, int M, int N, int K,
                                                                  void *__restrict__ C, Epi epi, uint32_t *part,
                                                                  int tile_base, int n_main)
{
    constexpr int kWN = kBN / 2;  // a wave's columns
    constexpr int kTJ = kWN / 32; // its 32-wide column tiles
    __shared__ __attribute__((aligned(1024))) uint8_t st0[kPTStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[kPTStageBytes];
    // MXFP8: the scale dwords of an even and of an odd group of four slices
    // (two LDS objects, like the stages), each A rows' then B rows' [row][4]
    // with one dword of padding after every 16 rows: row r's dword d sits at
    // 4 r + r / 16 + d, so the 32 rows a scale read touches (fr = 0..31) fall
    // in 32 different banks
    constexpr int kSxGroup = 2 * kBM * 4 + 2 * kBM / 16;
    __shared__ __attribute__((aligned(16))) uint32_t sxe[kMX ? kSxGroup : 1];
    __shared__ __attribute__((aligned(16))) uint32_t sxo[kMX ? kSxGroup : 1];
    __shared__ uint32_t red[kGemmThreads / 64];
    constexpr int kStageLoads = 8 + kBN / 32; // direct loads per lane per stage

    int tm, tn;
    const int tilesM = (M + kBM - 1) / kBM, tilesN = (N + kBM - 1) / kBM;
    if constexpr (kBN == kBM) group_tile(xcd_order(blockIdx.x, n_main), tilesM, tilesN, tm, tn);
    else group_tile(tile_base + (int)(blockIdx.x >> 1), tilesM, tilesN, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBM + (kBN == kBM ? 0 : (blockIdx.x & 1) * kBN);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int fr = lane & 31, fg = lane >> 5;
    const int nk = K / kBK;

    const int64_t a_rows = min((int64_t)kBM, (int64_t)M - m0), b_rows = min((int64_t)kBN, (int64_t)N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)(A + m0 * K), 0, (int)(a_rows * K), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void *)(B + n0 * K), 0, (int)(b_rows * K), kRawBufferWord3);
    // lane L of a 1 KiB load writes physical chunk L % 8 of row 8(w + 4u) + L / 8,
    // which holds logical chunk (L % 8) ^ ((row >> 1) & 7) = (L % 8) ^ ((4w + L / 16) & 7)
    const int voff = (lane >> 3) * K + (((lane & 7) ^ ((4 * w + (lane >> 4)) & 7)) << 4);

    // MXFP8 scale rows: K/32 bytes per row; the slice's 4 bytes are one dword
    const int kx = K / 32;
    const __amdgpu_buffer_rsrc_t rxa = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint8_t *>(sA) + (kMX ? m0 * kx : 0)), 0, kMX ? (int)(a_rows * kx) : 4,
        kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rxb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint8_t *>(sB) + (kMX ? n0 * kx : 0)), 0, kMX ? (int)(b_rows * kx) : 4,
        kRawBufferWord3);

    // wave w loads rows 8(w + 4u), u = 0..7, of the A panel and u < kBN / 32
    // of the B panel (16 or 12 loads of 1 KiB)
    auto stage = [&](uint8_t *st, int kb) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int row = 8 * (w + 4 * u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(st + row * kBK), 16, voff, row * K + kb * kBK,
                                                     0, 0);
            if (u < kBN / 32)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(st + kBM * kBK + row * kBK), 16, voff,
                                                         row * K + kb * kBK, 0, 0);
        }
    };
    // MXFP8 scale group g (slices 4g .. 4g+3) into sxe (g even) or sxo (g odd):
    // wave w loads rows 64w .. 64w+63 of both panels, 16 rows per load (one
    // padded run of 64 dwords), lane L the dword L % 4 of row L / 4 (bytes past
    // a panel read zero; bytes past a row's last slice, of groups past the last
    // one too, are never read)
    const int sx_voff = (lane >> 2) * kx + 4 * (lane & 3);
    constexpr int kScaleGroupLoads = 8; // loads per lane per scale group
    auto sx_pos = [](int r) { return 4 * r + (r >> 4); };
    auto scale_group_to = [&](uint32_t *dst, int g) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 64 * w + 16 * q;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rxa, (lds_void *)(dst + sx_pos(row)), 4, sx_voff,
                                                     row * kx + 16 * g, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rxb, (lds_void *)(dst + sx_pos(kBM + row)), 4, sx_voff,
                                                     row * kx + 16 * g, 0, 0);
        }
    };
    auto scale_group = [&](int g, bool odd) {
        if constexpr (kMX) scale_group_to(odd ? sxo : sxe, g);
    };

    v16f acc[4][kTJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    v8i fa0[4], fb0[kTJ], fa1[4], fb1[kTJ]; // first-half and second-half fragments
    // MXFP8: the scale dwords of the lane's A rows (i) and B rows (j) for the
    // current slice and the next one, pre-shifted by 8 * fg bytes so that byte
    // 0 is the scale of this lane's K block in half 0 and byte 2 in half 1
    uint32_t xa0[4], xb0[kTJ], xa1[4], xb1[kTJ];
    auto read_frags = [&](const uint8_t *st, int h, v8i(&a)[4], v8i(&b)[kTJ]) {
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
            b[j] = kMX ? read_frag32_mx(st + kBM * kBK, wn * kWN + 32 * j + fr, fg, h)
                       : read_frag32(st + kBM * kBK, wn * kWN + 32 * j + fr, fg, h);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = kMX ? read_frag32_mx(st, wm * 128 + 32 * i + fr, fg, h) : read_frag32(st, wm * 128 + 32 * i + fr, fg, h);
    };
    // the scale dwords of slice kb (group kb / 4, dword kb % 4 of each row)
    auto read_scales_from = [&](const uint32_t *sx, uint32_t(&xa)[4], uint32_t(&xb)[kTJ]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = sx[sx_pos(wm * 128 + 32 * i + fr)] >> (8 * fg);
#pragma unroll
        for (int j = 0; j < kTJ; ++j) xb[j] = sx[sx_pos(kBM + wn * kWN + 32 * j + fr)] >> (8 * fg);
    };
    // (odd: the group of slice kb is odd, so its dwords are in sxo)
    auto read_scales = [&](int kb, bool odd, uint32_t(&xa)[4], uint32_t(&xb)[kTJ]) {
        if constexpr (kMX) read_scales_from((odd ? sxo : sxe) + (kb & 3), xa, xb);
    };
    // half h of the slice whose scale dwords are xa / xb
    auto mfmas = [&](const v8i(&a)[4], const v8i(&b)[kTJ], const uint32_t(&xa)[4], const uint32_t(&xb)[kTJ], int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < kTJ; ++j) {
                if constexpr (kMX) {
                    if (h == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], FB, FA, 0,
                                                                                    (int)xb[j], 0, (int)xa[i]);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], FB, FA, 2,
                                                                                    (int)xb[j], 2, (int)xa[i]);
                } else {
                    acc[i][j] = mfma32x32x64<FB, FA>(b[j], a[i], acc[i][j]);
                }
            }
    };

    // One slice in stage `cur` (the next one in `nxt`).  `full` = the slices
    // kb + 1 and kb + 2 both exist (no guards).
    // MXFP8: slice kb = 8t + p has a fixed place p in the unrolled loop.  At
    // p = 0 and 4 (the first slice of group g) it loads group g + 1 at its end
    // (into the object group g is not in).  Those loads are then the youngest
    // of the wave, and the wait of the next slice (p = 1, 5) lets them stay in
    // flight; that slice reads only group g's object, so the compiler's wait
    // insertion keeps the two apart.  The slice after it issues loads of its
    // own, so its wait (like every other) is a full one: the group has about
    // a slice and a half to arrive instead of half a slice.
    auto slice = [&](int kb, int p, uint8_t *cur, const uint8_t *nxt, const uint32_t(&xa)[4],
                     const uint32_t(&xb)[kTJ], uint32_t(&xan)[4], uint32_t(&xbn)[kTJ], bool full) {
        const bool issue = kMX && (p & 3) == 0, relaxed = kMX && (p & 3) == 1;
        // half 0
        mfmas(fa0, fb0, xa, xb, 0);
        read_frags(cur, 1, fa1, fb1);
        if (full) {
#pragma unroll
            for (int t = 0; t < 4 * kTJ; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // LDS read
            }
        }
        // sync: the next slice landed (this lane's loads, then every wave's).
        // MXFP8: the scale group issued at the end of the previous slice (the
        // youngest kScaleGroupLoads loads) may stay in flight through this wait.
        // (scheduling barriers keep every matrix instruction on its side of the
        // slice barrier; the scheduler otherwise moves some across it, and in
        // the MXFP8 eight-slice loop the halves lose their balance)
        __builtin_amdgcn_sched_barrier(0);
        if (relaxed)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(kScaleGroupLoads, 0));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // half 1: the next slice's scales first, while no direct load is in
        // flight (the scale buffers are one LDS object whose group is chosen
        // at run time, and the compiler's wait insertion would otherwise hold
        // the reads for the stage loads issued below)
        if (full || kb + 1 < nk) read_scales(kb + 1, (((p + 1) >> 2) & 1) != 0, xan, xbn);
        if (full || kb + 2 < nk) stage(cur, kb + 2);
        mfmas(fa1, fb1, xa, xb, 1);
        if (full || kb + 1 < nk) read_frags(nxt, 0, fa0, fb0);
        if (full) {
#pragma unroll
            for (int t = 0; t < 4 * kTJ; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // LDS read
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // global -> LDS load
            }
        }
        // MXFP8: at the first slice of group g, group g + 1 goes into the
        // object whose last reads (slice 4g - 1's scales, read during slice
        // 4g - 2) every wave finished before this slice's barrier; its first
        // reader is slice 4g + 3, after full waits.  Loaded also past the last
        // group (reading zeros or unused bytes), so that the relaxed wait of
        // the next slice holds in every tile.
        if (issue) scale_group((kb >> 2) + 1, ((p >> 2) & 1) == 0);
    };

    // prologue: slices 0 and 1 in flight, slice 0's first-half fragments.
    // Both stages are always filled (for K = 128 the second load reads bytes
    // of the panel that are never used; rows past the record read zero): with
    // an unconditional pair the compiler's wait insertion keeps the two stages
    // apart and puts no full wait at the top of the loop.
    if (nk > 0) {
        scale_group(0, false);
        stage(st0, 0);
        stage(st1, 1);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kStageLoads, 15));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        read_frags(st0, 0, fa0, fb0);
        read_scales(0, false, xa0, xb0);
    }
    int kb = 0;
    if constexpr (kMX) {
        // eight slices per trip, so that every slice's place, and with it its
        // wait and the scale object it reads, is fixed at compile time
        for (; kb + 10 <= nk; kb += 8) {
            slice(kb, 0, st0, st1, xa0, xb0, xa1, xb1, true);
            slice(kb + 1, 1, st1, st0, xa1, xb1, xa0, xb0, true);
            slice(kb + 2, 2, st0, st1, xa0, xb0, xa1, xb1, true);
            slice(kb + 3, 3, st1, st0, xa1, xb1, xa0, xb0, true);
            slice(kb + 4, 4, st0, st1, xa0, xb0, xa1, xb1, true);
            slice(kb + 5, 5, st1, st0, xa1, xb1, xa0, xb0, true);
            slice(kb + 6, 6, st0, st1, xa0, xb0, xa1, xb1, true);
            slice(kb + 7, 7, st1, st0, xa1, xb1, xa0, xb0, true);
        }
        // at most nine slices remain; kb % 8 == 0
        if (kb < nk) slice(kb, 0, st0, st1, xa0, xb0, xa1, xb1, false);
        if (kb + 1 < nk) slice(kb + 1, 1, st1, st0, xa1, xb1, xa0, xb0, false);
        if (kb + 2 < nk) slice(kb + 2, 2, st0, st1, xa0, xb0, xa1, xb1, false);
        if (kb + 3 < nk) slice(kb + 3, 3, st1, st0, xa1, xb1, xa0, xb0, false);
        if (kb + 4 < nk) slice(kb + 4, 4, st0, st1, xa0, xb0, xa1, xb1, false);
        if (kb + 5 < nk) slice(kb + 5, 5, st1, st0, xa1, xb1, xa0, xb0, false);
        if (kb + 6 < nk) slice(kb + 6, 6, st0, st1, xa0, xb0, xa1, xb1, false);
        if (kb + 7 < nk) slice(kb + 7, 7, st1, st0, xa1, xb1, xa0, xb0, false);
        if (kb + 8 < nk) slice(kb + 8, 0, st0, st1, xa0, xb0, xa1, xb1, false);
    } else {
        for (; kb + 4 <= nk; kb += 2) {
            slice(kb, 0, st0, st1, xa0, xb0, xa1, xb1, true);
            slice(kb + 1, 1, st1, st0, xa1, xb1, xa0, xb0, true);
        }
        // at most three slices remain; kb is even
        if (kb < nk) slice(kb, 0, st0, st1, xa0, xb0, xa1, xb1, false);
        if (kb + 1 < nk) slice(kb + 1, 1, st1, st0, xa1, xb1, xa0, xb0, false);
        if (kb + 2 < nk) slice(kb + 2, 0, st0, st1, xa0, xb0, xa1, xb1, false);
    }

    // epilogue: lane (fr, fg) of 32x32 tile (i, j) holds C[row][4 consecutive
    // columns 8q + 4fg .. +3] for q = 0..3
    const float alpha = kMX ? 1.0f : (*sA) * (*sB);
    const float out_scale = kOut >= kOutE4M3 ? 1.0f / *epi.out_si : 0.0f;
    uint32_t m = 0;
    {
        // M and N are multiples of 128: a wave's sub-tile is wholly inside C
        // or wholly outside.  Two waves share each 64 KiB stage.
        typedef EpiStage<kWN, out_bytes<kOut>(), 128, kPTStageBytes / 2> ES;
        const int64_t wrow0 = m0 + wm * 128, wcol0 = n0 + wn * kWN;
        const bool inside = wrow0 < M && wcol0 < N;
        uint8_t *ep = (w < 2 ? st0 : st1) + (w & 1) * (kPTStageBytes / 2);
#pragma unroll
        for (int ps = 0; ps < ES::kPasses; ++ps) {
            __syncthreads(); // the stages (then the previous pass) are no longer read
            if (inside) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if ((32 * i) / ES::kPassRows != ps) continue;
#pragma unroll
                    for (int j = 0; j < kTJ; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const v4f v = v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                              acc[i][j][4 * q + 3]} * alpha;
                            const uint4 bits =
                                pack_out4<kOut, kAmax, kFuse>(wcol0 + 32 * j + 8 * q + 4 * fg, v, m, epi, out_scale);
                            ES::put(ep, 32 * i + fr - ps * ES::kPassRows, 8 * j + 2 * q + fg, bits);
                        }
                }
            }
            __syncthreads();
            if (inside) ES::store(ep, C, N, wrow0 + ps * ES::kPassRows, wcol0, lane);
        }
    }
    if constexpr (kAmax) {
        m = block_max_u32<kGemmThreads>(m, red);
        if (tid == 0) atomicMax(&part[blockIdx.x % kParts], canonical_amax_bits(m));
    }
}

// ---------------------------------------------------------------------------
// Block-scaled kernel.  A 256 x kBN block tile (kBN = 256; 128 for the half
// tiles of a last, partly empty round), eight waves (4 x 2) of 64 x kBN/2,
// each as 4 x kBN/32 tiles of 16x16.  One K step is one 128-wide scale slice
// and one v_mfma_f32_16x16x128_f8f6f4 per tile, started from zero, so its
// result is exactly that slice's partial product; it is promoted at once,
//   acc = fma(part, fl32(sA[row][kb] * sB[col block or col][kb]), acc),
// with the accumulators in ordinary vector registers (the vector ALU cannot
// operate on AGPRs; 128 per lane for full tiles, within the budget of two
// waves per SIMD).
//
// Ping-pong schedule.  The waves form two groups, X (waves 0-3) and Y (waves
// 4-7), one wave of each on every SIMD, and a slice runs as four phases
// separated by barriers: in each phase one group computes half of its slice
// (its first or second kBN/64 column tiles: the MFMAs, each followed by the
// promotion of the tile two before it) from fragments already in registers,
// while the other group reads its next fragments from LDS, finishes the
// promotion of its last two tiles and issues global loads.  So every SIMD
// always has one wave feeding its matrix pipe while the other waits on
// memory, instead of both waves stalling together at one barrier per slice
// (measured on the MI355X, fprop 4096x14336x4096: the matrix pipes are busy
// 0.62 of the active cycles, against 0.46 with that lockstep schedule).
//
// Memory: two stages (A rows 0..255 and B rows 0..kBN-1 of one slice) plus
// per-stage scales.  Every wave loads an eighth of each, in two groups per
// slice, each in one of its read phases: group 1 (A, the B rows that both
// groups read first, the A row scales and B's scales) once the stage's
// previous A and first-half B reads are over, group 2 (the B rows read
// second) once its second-half reads are over, at least five phases before
// they are read.  Every wave issues the same loads in the same order, so one
// vmcnt threshold at the end of every phase (G1 + G2 younger loads
// outstanding) proves that the data the next phases read has landed.
constexpr int kBSThreads = 512;

template <int kv> struct PhaseC {
    static constexpr int value = kv;
};

template <int FA, int FB, bool kAmax, int kOut, bool kFuse, bool kRowB, int kBN>
__global__ __launch_bounds__(kBSThreads, 1) void gemm_bs_pp_kernel(const uint8_t *__restrict__ A,
                                                                   const uint8_t *__restrict__ B,
                                                                   const float *__restrict__ sA,
                                                                   const float *__restrict__ sB, int M, int N, int K,
                                                                   void *__restrict__ C, Epi epi, uint32_t *part,
                                                                   int tile_base, int n_main)
{
    // One LDS object per stage (the compiler's wait insertion tells the direct
    // loads into different objects apart, so a read of one stage never waits
    // for the loads landing in the other; within a stage the loads that a
    // read does not need were issued four phases earlier).  Stage layout:
    //   A      rows 0..255 of the tile (32 KiB)
    //   B0     the B rows each wave reads first: tile rows 0..Q-1 (group X)
    //          then 2Q..3Q-1 (group Y), Q = kBN / 4 (2Q rows)
    //   B1     the B rows each wave reads second: Q..2Q-1, then 3Q..4Q-1
    //   SA     the slice's 256 A row scales
    //   SB0    1x128 B: the scales of B0's rows; 128x128 B: the block scales
    //          of the tile's column blocks at [0], [1] (each loading wave
    //          writes a 64-float copy)
    //   SB1    1x128 B: the scales of B1's rows
    // B row n of the tile is row (n / 2Q) * Q + n % Q of B0 (n % 2Q < Q) or
    // B1.  Rows are 128 bytes with 16-byte chunks XOR-swizzled by row.
    constexpr int kQ = kBN / 4, kJT = kQ / 16;         // a half's columns and 16-wide column tiles
    constexpr int kAB = kBM * kBK, kB2 = 2 * kQ * kBK; // code bytes of A, of B0 / B1
    constexpr int oB0 = kAB, oB1 = kAB + kB2, oSA = kAB + 2 * kB2, oSB0 = oSA + 4 * kBM, oSB1 = oSB0 + 4 * kBM;
    constexpr int kStage = oSB1 + 2 * kBM;
    __shared__ __attribute__((aligned(1024))) uint8_t st0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[kStage];
    __shared__ uint32_t red[kBSThreads / 64];
    constexpr int kBL = kBN / 128;         // loads per wave of one B half
    constexpr int G1 = 4 + kBL + 1;        // loads per wave in group 1
    constexpr int G2 = kBL + (kRowB ? 1 : 0); // and in group 2
    constexpr int kVm = G1 + G2;           // younger loads allowed at the end of every phase
    auto fptr = [](uint8_t *st, int off) { return reinterpret_cast<float *>(st + off); };

    // kBN = 256: grid block b -> grouped tile xcd_order(b, n_main).  kBN =
    // 128: half b & 1 (columns 128 (b & 1) ..) of grouped tile tile_base + b / 2
    int tm, tn;
    const int tilesM = (M + kBM - 1) / kBM, tilesN = (N + kBM - 1) / kBM;
    if constexpr (kBN == kBM) group_tile(xcd_order(blockIdx.x, n_main), tilesM, tilesN, tm, tn);
    else group_tile(tile_base + (int)(blockIdx.x >> 1), tilesM, tilesN, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBM + (kBN == kBM ? 0 : (blockIdx.x & 1) * kBN);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool gx = w < 4;
    const int wm = w & 3, wn = w >> 2; // rows 64 wm .., columns 2Q wn .. of the tile
    const int fr = lane & 15, fg = lane >> 4;
    const int kblocks = K / kBK;

    const int64_t a_rows = min((int64_t)kBM, (int64_t)M - m0), b_rows = min((int64_t)kBN, (int64_t)N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)(A + m0 * K), 0, (int)(a_rows * K), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void *)(B + n0 * K), 0, (int)(b_rows * K), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)(sA + m0 * kblocks), 0,
                                                                        (int)(a_rows * kblocks * 4), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rsb =
        kRowB ? __builtin_amdgcn_make_buffer_rsrc((void *)(sB + n0 * kblocks), 0, (int)(b_rows * kblocks * 4),
                                                  kRawBufferWord3)
              : __builtin_amdgcn_make_buffer_rsrc((void *)sB, 0, (int)((N / 128) * kblocks * 4), kRawBufferWord3);
    // Every wave loads an eighth of each region: rows 8(w + 8u) + L / 8; lane L
    // writes physical chunk L % 8 of its row, which holds logical chunk
    // (L % 8) ^ ((row >> 1) & 7) = (L % 8) ^ ((4 w + L / 16) & 7)
    const int voff = (lane >> 3) * K + (((lane & 7) ^ ((4 * w + (lane >> 4)) & 7)) << 4);
    // 128x128 B: lanes 0 and 1 fetch the scales of the tile's two column
    // blocks (clamped inside B for a tile column past N, whose results are
    // never stored), the other lanes repeat them.  1x128 B: lane L fetches the
    // scale of LDS row lrow + L of B0, lrow = 64 (w & 1) when B0 has 128 rows.
    const int sb_lrow = kBN == kBM ? 64 * (w & 1) : 0;
    const int sb_voff = kRowB ? (((sb_lrow + lane) / kQ) * 2 * kQ + (sb_lrow + lane) % kQ) * kblocks * 4
                              : min((int)(n0 / 128) + (lane & 1), N / 128 - 1) * kblocks * 4;

    // A: rows 8(w + 8u), u = 0..3; B half h: LDS rows 8(w + 8u), u < kBL,
    // holding tile rows (LDS row / Q) * 2Q + Q h + LDS row % Q
    auto load_a = [&](uint8_t *dst, int kb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 8 * (w + 8 * u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(dst + row * kBK), 16, voff, row * K + kb * kBK,
                                                     0, 0);
        }
    };
    auto load_b = [&](uint8_t *dst, int h, int kb) {
#pragma unroll
        for (int u = 0; u < kBL; ++u) {
            const int row = 8 * (w + 8 * u);
            const int trow = (row / kQ) * 2 * kQ + kQ * h + row % kQ;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(dst + row * kBK), 16, voff, trow * K + kb * kBK,
                                                     0, 0);
        }
    };
    // 1x128 B: the scales of half h's LDS rows sb_lrow .. + 63 (the waves
    // that load the same rows write the same values)
    auto load_sb_rows = [&](float *dst, int h, int kb) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void *)(dst + sb_lrow), 4, sb_voff,
                                                 (kQ * h * kblocks + kb) * 4, 0, 0);
    };
    // group 1 of slice kb: A, B's first half, and one scale load per wave
    // (waves 0-3: A row scales 64 w ..; waves 4-7: B's first-half scales)
    auto load_g1 = [&](uint8_t *st, int kb) {
        load_a(st, kb);
        load_b(st + oB0, 0, kb);
        if (w < 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(st + oSA + 4 * 64 * w), 4, lane * kblocks * 4,
                                                     (64 * w * kblocks + kb) * 4, 0, 0);
        else if constexpr (kRowB)
            load_sb_rows(fptr(st, oSB0), 0, kb);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void *)(st + oSB0 + 4 * 64 * (w - 4)), 4, sb_voff,
                                                     kb * 4, 0, 0);
    };
    // group 2 of slice kb: B's second half (and its 1x128 scales)
    auto load_g2 = [&](uint8_t *st, int kb) {
        load_b(st + oB1, 1, kb);
        if constexpr (kRowB) load_sb_rows(fptr(st, oSB1), 1, kb);
    };

    v4f acc[4][2 * kJT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2 * kJT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    v8i a[4], b[kJT]; // the slice's A fragments, the half's B fragments
    float wi[4];      // 128x128 B: weight of row i; 1x128 B: sA of row i
    v4f sbq[kJT];     // 1x128 B: the half's column scales, per 16-column tile
    v4f pr[3];        // MFMA results awaiting promotion (tile t in pr[t % 3])

    // weight of tile (i, column tile jj of the half) for element e
    auto weight = [&](int i, int jj, int e) { return kRowB ? wi[i] * sbq[jj][e] : wi[i]; };
    // promote tile t (t = 4 jj + i) of half h
    auto promote = [&](auto hc, int t) {
        constexpr int h = decltype(hc)::value;
        const int i = t & 3, jj = t >> 2;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[i][kJT * h + jj][e] = __builtin_fmaf(pr[t % 3][e], weight(i, jj, e), acc[i][kJT * h + jj][e]);
        // keeps these FMAs in their phase (ordered with the phase boundary's
        // volatile statements)
        asm volatile("" : "+v"(acc[i][kJT * h + jj]));
    };
    // compute phase of half h: MFMA of tile t, then the promotion of tile t - 2
    // (its result has landed); the last two tiles are promoted by the next phase
    constexpr int kT = 4 * kJT;
    auto compute = [&](auto hc) {
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            pr[t % 3] = mfma16x16x128<FB, FA>(b[t >> 2], a[t & 3], v4f{0.f, 0.f, 0.f, 0.f});
            if (t >= 2) promote(hc, t - 2);
        }
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
            if (t >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0); // promotion FMAs
        }
    };
    auto tail = [&](auto hc) {
        promote(hc, kT - 2);
        promote(hc, kT - 1);
    };
    auto read_a = [&](const uint8_t *st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = read_frag(st, wm * 64 + 16 * i + fr, fg);
    };
    auto read_b = [&](const uint8_t *st) {
#pragma unroll
        for (int jj = 0; jj < kJT; ++jj) b[jj] = read_frag(st, wn * kQ + 16 * jj + fr, fg);
    };
    // the slice's weights (with the first half) and the half's 1x128 column scales
    auto read_scales = [&](const float *ssa_, const float *ssbh, int h) {
        if (h == 0) {
            if constexpr (kRowB) {
#pragma unroll
                for (int i = 0; i < 4; ++i) wi[i] = ssa_[wm * 64 + 16 * i + fr];
            } else {
                // a wave's 2Q columns lie in column block wn of a full tile,
                // in the one block of a half tile
                const float sb = ssbh[kBN == kBM ? wn : 0];
#pragma unroll
                for (int i = 0; i < 4; ++i) wi[i] = ssa_[wm * 64 + 16 * i + fr] * sb;
            }
        }
        if constexpr (kRowB) {
#pragma unroll
            for (int jj = 0; jj < kJT; ++jj)
                sbq[jj] = *reinterpret_cast<const v4f *>(ssbh + wn * kQ + 16 * jj + 4 * fg);
        }
    };
    // Phase boundaries.  The scheduling barriers keep every instruction on
    // its side (matrix and vector instructions touch no memory, so a memory
    // fence alone would let them drift across the barrier into the other
    // phase); the end of a read phase waits for its LDS reads, the end of a
    // compute phase for the loads the next phases read.
    auto phase_end = [&](auto wc) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(decltype(wc)::value);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto sync_lds = [&]() { phase_end(PhaseC<waitcnt_imm(kVm, 0)>{}); };
    auto sync = [&]() { phase_end(PhaseC<waitcnt_imm(kVm, 15)>{}); };
    using H0 = PhaseC<0>;
    using H1 = PhaseC<1>;

    // One slice (stage cur, the other stage nxt): four operations, one per
    // phase, each ending at a barrier after the wave has waited for all but
    // its kVm youngest loads.  Group X runs the operations one phase ahead of
    // group Y, so in every phase one group computes while the other reads.
    // Each wave loads in its read phases: in M0 its share of group 2 of the
    // next slice into nxt (both groups have read nxt's second-half B by then),
    // in M1 its share of group 1 of slice kb + 2 into cur (both have read its A
    // and first-half B).  Data is read at least five phases after it was
    // requested, and every wave issues the same loads in every slice (loads
    // past the last slice read bytes that are never used, or zeros past the
    // panel), so the one threshold holds in every phase.
    auto slice = [&](int kb, uint8_t *cur, uint8_t *nxt) {
        read_a(cur); // M0: A and the first half's B fragments, the slice's weights
        read_b(cur + oB0);
        tail(H1{});
        read_scales(fptr(cur, oSA), fptr(cur, oSB0), 0);
        load_g2(nxt, kb + 1);
        sync_lds();
        compute(H0{}); // C0
        sync();
        read_b(cur + oB1); // M1
        tail(H0{});
        read_scales(fptr(cur, oSA), fptr(cur, oSB1), 1);
        load_g1(cur, kb + 2);
        sync_lds();
        compute(H1{}); // C1
        sync();
    };

    // prologue: groups 1 and 2 of slice 0 and group 1 of slice 1 (slice 0's
    // first read phase loads group 2 of slice 1), then slice 0's group 1 landed
    if (kblocks > 0) {
        load_g1(st0, 0);
        load_g2(st0, 0);
        load_g1(st1, 1);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(G2 + G1, 15));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // nothing to promote yet: zero partials and weights make the first
    // tail a no-op
#pragma unroll
    for (int q = 0; q < 3; ++q) pr[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) wi[i] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kJT; ++jj) sbq[jj] = v4f{0.f, 0.f, 0.f, 0.f};
    if (!gx) sync(); // group Y starts one phase later
    int kb = 0;
    for (; kb + 1 < kblocks; kb += 2) {
        slice(kb, st0, st1);
        slice(kb + 1, st1, st0);
    }
    if (kb < kblocks) slice(kb, st0, st1);
    if (gx) sync(); // and ends one phase later
    tail(H1{});
    // the loads of the slices past the end must land before the stages are reused
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // epilogue: lane (fr, fg) of tile (i, j) holds C[row][4 consecutive cols];
    // each wave stages its 64 x 2Q results in kB2 bytes of the freed stages
    const float out_scale = kOut >= kOutE4M3 ? 1.0f / *epi.out_si : 0.0f;
    uint32_t m = 0;
    {
        typedef EpiStage<2 * kQ, out_bytes<kOut>(), 64, kB2> ES;
        const int64_t wrow0 = m0 + wm * 64, wcol0 = n0 + wn * 2 * kQ;
        const bool inside = wrow0 < M && wcol0 < N;
        uint8_t *ep = (w < 4 ? st0 : st1) + (w & 3) * kB2;
#pragma unroll
        for (int ps = 0; ps < ES::kPasses; ++ps) {
            __syncthreads(); // the stages (then the previous pass) are no longer read
            if (inside) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if ((16 * i) / ES::kPassRows != ps) continue;
#pragma unroll
                    for (int j = 0; j < 2 * kJT; ++j) {
                        const uint4 bits =
                            pack_out4<kOut, kAmax, kFuse>(wcol0 + 16 * j + 4 * fg, acc[i][j], m, epi, out_scale);
                        ES::put(ep, 16 * i + fr - ps * ES::kPassRows, 4 * j + fg, bits);
                    }
                }
            }
            __syncthreads();
            if (inside) ES::store(ep, C, N, wrow0 + ps * ES::kPassRows, wcol0, lane);
        }
    }
    if constexpr (kAmax) {
        m = block_max_u32<kBSThreads>(m, red);
        if (tid == 0) atomicMax(&part[blockIdx.x % kParts], canonical_amax_bits(m));
    }
}

inline int gemm_grid(int64_t M, int64_t N) { return (int)(((M + kBM - 1) / kBM) * ((N + kBM - 1) / kBM)); }

template <int FA, int FB, int kOut, bool kFuse>
hipError_t launch_gemm_epi(const GemmArgs &a)
{
    const int m = (int)a.M, n = (int)a.N, k = (int)a.K;
    const Epi epi{a.bias, a.act, a.out_scale_inv};
    // A last wave of tiles that is at most half full runs as a full wave of
    // half tiles (256x128), launched after the full tiles.
    const int tiles = gemm_grid(a.M, a.N), r = a.cus > 0 ? tiles % a.cus : 0;
    const int n_main = (r > 0 && 2 * r <= a.cus) ? tiles - r : tiles;
    const int n_half = 2 * (tiles - n_main);
    uint32_t *part = a.gs ? a.gs->part : nullptr;
    if (a.mode == 0 || a.mode == 3) {
#define FP8Q_PT_LAUNCH(FLAG, BN, GRID, PART, BASE)                                                                  \
        do {                                                                                                        \
            if (a.amax_out)                                                                                         \
                gemm_pt_kernel<FA, FB, true, kOut, kFuse, FLAG, BN><<<GRID, kGemmThreads, 0, a.stream>>>(           \
                    a.A, a.B, a.sA, a.sB, m, n, k, a.C, epi, PART, BASE, n_main);                                   \
            else                                                                                                    \
                gemm_pt_kernel<FA, FB, false, kOut, kFuse, FLAG, BN><<<GRID, kGemmThreads, 0, a.stream>>>(          \
                    a.A, a.B, a.sA, a.sB, m, n, k, a.C, epi, PART, BASE, n_main);                                   \
        } while (0)
        if (a.mode == 0) {
            if (n_main > 0) FP8Q_PT_LAUNCH(false, kBM, n_main, part, 0);
            if (n_half > 0) FP8Q_PT_LAUNCH(false, kBM / 2, n_half, part, n_main);
        } else {
            if (n_main > 0) FP8Q_PT_LAUNCH(true, kBM, n_main, part, 0);
            if (n_half > 0) FP8Q_PT_LAUNCH(true, kBM / 2, n_half, part, n_main);
        }
#undef FP8Q_PT_LAUNCH
    } else {
#define FP8Q_BS_PP_LAUNCH(ROWB, BN, GRID, BASE)                                                                     \
        do {                                                                                                        \
            if (a.amax_out)                                                                                         \
                gemm_bs_pp_kernel<FA, FB, true, kOut, kFuse, ROWB, BN><<<GRID, kBSThreads, 0, a.stream>>>(          \
                    a.A, a.B, a.sA, a.sB, m, n, k, a.C, epi, part, BASE, n_main);                                   \
            else                                                                                                    \
                gemm_bs_pp_kernel<FA, FB, false, kOut, kFuse, ROWB, BN><<<GRID, kBSThreads, 0, a.stream>>>(         \
                    a.A, a.B, a.sA, a.sB, m, n, k, a.C, epi, part, BASE, n_main);                                   \
        } while (0)
        if (a.mode == 1) {
            if (n_main > 0) FP8Q_BS_PP_LAUNCH(false, kBM, n_main, 0);
            if (n_half > 0) FP8Q_BS_PP_LAUNCH(false, kBM / 2, n_half, n_main);
        } else {
            if (n_main > 0) FP8Q_BS_PP_LAUNCH(true, kBM, n_main, 0);
            if (n_half > 0) FP8Q_BS_PP_LAUNCH(true, kBM / 2, n_half, n_main);
        }
#undef FP8Q_BS_PP_LAUNCH
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.amax_out) return e;
    // blocks b of both launches folded into part[b % kParts]
    return launch_finish_amax(a.gs, n_main > kParts || n_half > kParts ? kParts : (n_main > n_half ? n_main : n_half),
                              a.amax_out, a.stream);
}

// Every output kind and epilogue of one operand-format pair.  The plain
// epilogue (no bias, no activation) is its own instantiation, so the GEMM
// without fusions is compiled exactly as if the fused code did not exist; an
// FP8 output always takes the fused epilogue.
template <int FA, int FB>
hipError_t launch_gemm_pair(const GemmArgs &a)
{
    const bool fuse = a.bias != nullptr || a.act != kActNone;
    switch (a.out_kind) {
    case kOutF32:
        return fuse ? launch_gemm_epi<FA, FB, kOutF32, true>(a) : launch_gemm_epi<FA, FB, kOutF32, false>(a);
    case kOutE4M3: return launch_gemm_epi<FA, FB, kOutE4M3, true>(a);
    case kOutE5M2: return launch_gemm_epi<FA, FB, kOutE5M2, true>(a);
    default:
        return fuse ? launch_gemm_epi<FA, FB, kOutBF16, true>(a) : launch_gemm_epi<FA, FB, kOutBF16, false>(a);
    }
}

} // namespace fp8q

#endif // FP8Q_GEMM_KERNELS_H
