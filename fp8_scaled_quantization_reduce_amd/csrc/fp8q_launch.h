// fp8q_launch.h -- internal launchers behind the C ABI.  Arguments are
// already validated by the API layer; each launcher only enqueues kernels on
// `s` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Grid-wide reduction scratch.  A flat or tile kernel that reduces an amax
// runs at most kParts producing blocks (grid-stride loops cover larger
// inputs).  When the launch ends in its own finishing block (the amax, the
// casts with output amax and the delayed step), block b publishes its
// canonical magnitude max to pub[b] tagged with the call's tag (tag << 32 |
// bits), and the finishing block waits until all pub[0 .. nblocks) carry the
// tag, then puts them back to zero (a partial that arrives after its
// finishing block gave up carries a tag that no later call accepts).
// Otherwise block b stores its max to part[b], a GEMM block folds its max into
// part[b % kParts] with an unsigned atomic max (the canonical magnitude bits
// order like the values, and the canonical NaN sorts above +inf), the cast
// statistics add each block's four counts into cnt[k][b % kCntParts], and one
// small kernel follows that reads the slots the call used, writes the result
// and puts them back to zero, so part and cnt are all zeros between calls
// (they start zeroed, as a device global).
#ifndef FP8Q_REDUCE_GRID
#define FP8Q_REDUCE_GRID 1024
#endif
constexpr int kParts = FP8Q_REDUCE_GRID;
constexpr int kCntParts = 64;
constexpr int kStats = 4; // overflows, underflows, NaNs, nonzeros
struct GridScratch {
    uint32_t part[kParts];
    unsigned long long cnt[kStats][kCntParts];
    unsigned long long pub[kParts];
};
static_assert(kParts % 256 == 0 && sizeof(GridScratch) == 12 * kParts + 2048, "scratch layout");

// A reducing call's scratch slot, its tag (nonzero and new for every call on
// the slot) and the bound on its finishing block's polling rounds.
struct Reduce {
    GridScratch *gs;
    uint32_t tag;
    uint32_t rounds;
};
// The default bound: about a second and more of polling.
constexpr uint32_t kPollRounds = 1u << 21;

// Flat launches that reduce nothing keep at most this many blocks.
#ifndef FP8Q_MAX_GRID
#define FP8Q_MAX_GRID 65536
#endif
constexpr int kMaxGrid = FP8Q_MAX_GRID;

// Scratch slots per device: one per stream that has run a reducing call.
constexpr int kScratchSlots = 64;

// Enqueue the zeroing of one scratch slot (after a failed call left it dirty).
hipError_t launch_clear_scratch(GridScratch *gs, hipStream_t s);

// Graphics clock of the CUs that run kClockBlocks one-wave blocks next to
// other work (consecutive blocks start on consecutive XCDs), from when the
// kernel starts until *stop is nonzero (at most kClockMonitorSeconds):
// out[3 b + 0, 1, 2] = XCD id, shader-clock cycles, constant-rate ticks of
// block b; out[3 kClockBlocks] = the constant rate in kHz.
constexpr int kClockBlocks = 8;
constexpr int kClockMonitorSeconds = 2;
hipError_t launch_clock_monitor(uint64_t *out, const uint32_t *stop, hipStream_t s);

// Where a per-tensor scale comes from: exactly one pointer is non-null.
struct ScaleSrc {
    const float *amax_in;      // current scaling from this amax
    const float *scale_inv_in; // a given dequant scale s
    int margin;                // current scaling only
};

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, hipStream_t s);

// Fold part[0 .. nparts) into *out and clear those slots.
hipError_t launch_finish_amax(GridScratch *gs, int nparts, float *out, hipStream_t s);

hipError_t launch_amax(const void *x, int dtype, int64_t n, float *amax, const Reduce &r, hipStream_t s);

// stats (nullable): uint64[4] counts of the cast, reduced in the same pass
hipError_t launch_cast(const void *x, int dtype, int64_t n, int fmt, ScaleSrc src, uint8_t *q, float *scale_inv_out,
                       float *scale_out, float *amax_out, uint64_t *stats, const Reduce &r, hipStream_t s);

hipError_t launch_dequant(const uint8_t *q, int fmt, int64_t n, const float *scale_inv, float *y, hipStream_t s);

hipError_t launch_rowwise_colwise(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, ScaleSrc src,
                                  uint8_t *q_row, uint8_t *q_col, float *scale_inv_out, float *scale_out,
                                  float *amax_out, const Reduce &r, hipStream_t s);

hipError_t launch_block(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, int block_rows, uint8_t *q_row,
                        float *s_row, uint8_t *q_col, float *s_col, hipStream_t s);

hipError_t launch_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t *q_row, uint8_t *s_row,
                     uint8_t *q_col, uint8_t *s_col, hipStream_t s);

hipError_t launch_hybrid(const void *x, int dtype, int64_t rows, int64_t cols, int row_fmt, int col_fmt,
                         int col_source, ScaleSrc src, ScaleSrc src_col, uint8_t *q_row, uint8_t *q_col,
                         float *row_scale_inv_out, float *col_scale_inv_out, float *amax_out, const Reduce &r,
                         hipStream_t s);

// Sub-quantizers of a per-direction quantization (values of the C ABI's
// FP8Q_SUBQ_*).
enum Subq { kSubqBlock128 = 0, kSubqBlock1x128 = 1, kSubqMX = 2, kSubqTensor = 3 };

// The rowwise copy by row_recipe in row_fmt and the columnwise copy by
// col_recipe in col_fmt, both from one pass over x; the columnwise copy is
// taken from x, or (col_from_rows) from the dequantized row codes.  A copy
// whose code pointer is null is skipped.  Scale buffers: float for the
// 128x128 and 1x128 blocks, E8M0 bytes for MXFP8, one float (the s used) for
// a per-tensor direction, whose scale comes from pt (at most one direction is
// per-tensor).
hipError_t launch_hybrid_blockwise(const void *x, int dtype, int64_t rows, int64_t cols, int row_recipe, int row_fmt,
                                   uint8_t *q_row, void *s_row, int col_recipe, int col_fmt, uint8_t *q_col,
                                   void *s_col, bool col_from_rows, ScaleSrc pt, hipStream_t s);

// stats[0..3] (uint64): overflows, underflows, NaNs, nonzeros of the cast of
// x with dequant scale *scale_inv.
hipError_t launch_cast_stats(const void *x, int dtype, int64_t n, int fmt, const float *scale_inv, uint64_t *stats,
                             GridScratch *gs, hipStream_t s);

hipError_t launch_error_feedback(const void *g, int dtype, float *residual, int64_t n, int fmt,
                                 const float *scale_inv, uint8_t *q, float *amax_out, const Reduce &r, hipStream_t s);

hipError_t launch_delayed(float *hist, int history_len, int n_cols, int col, const float *new_amax, int64_t step,
                          int fmt, int margin, int algo, float *scale, float *scale_inv, hipStream_t s);

hipError_t launch_delayed_step(const void *x, int dtype, int64_t n, int fmt, float *hist, int history_len, int n_cols,
                               int col, int64_t step, int fmt_next, int margin, int algo, float *scale,
                               float *scale_inv, uint8_t *q, float *q_scale_inv_out, float *amax_out, const Reduce &r,
                               hipStream_t s);

// out_kind: 0 bf16, 1 fp32, 2 E4M3FN codes, 3 E5M2 codes (cast with
// 1 / *out_scale_inv); act: 0 none, 1 ReLU, 2 GELU; bias [N] fp32 or null.
hipError_t launch_gemm(const uint8_t *A, int fa, const float *sA, const uint8_t *B, int fb, const float *sB, int64_t M,
                       int64_t N, int64_t K, int mode, void *C, int out_kind, const float *bias, int act,
                       const float *out_scale_inv, float *amax_out, GridScratch *gs, hipStream_t s);

} // namespace fp8q
