/*
 * fp8q.h -- C ABI of the FP8 scaled-quantization and scaled-FP8-GEMM library
 * (libfp8q.so, HIP kernels for gfx950 / MI355X).
 *
 * Pages cited (title, section):
 *   [MFP8]   "Megatron FP8" (sections 1-28)
 *   [HYBRID] "[Pytorch][Common] Hybrid quantization #2817" (TransformerEngine PR)
 *   [VIME]   "Low Precision Training and Rollout" (vime documentation)
 *
 * Conventions for every call below
 *  - All pointers are DEVICE memory owned by the caller, unless stated.  The
 *    library never copies device->host and never synchronises: each call
 *    enqueues its kernels on `stream` (a hipStream_t; NULL = the default
 *    stream) and returns.
 *  - The library never allocates device memory.  Calls that reduce over the
 *    whole grid (an amax, the cast statistics) keep per-block partials in a
 *    reduction scratch that is a device global of the library: 64 slots of
 *    14 KiB on each device, created with the library's code object on that
 *    device and held until the process ends.  Each stream gets a slot of its
 *    own the first time it runs such a call (a host-side table; no device
 *    work), so calls on different streams never share partials.  Either the
 *    call's finishing block (the last block of its reducing launch) waits for
 *    the other blocks' partials, which carry a tag new to the call, and
 *    puts the slots back to zero once it has them, or the call's last kernel
 *    reads the partials and clears them.  Either way the slot is left empty,
 *    so these calls can be captured in a HIP graph and replayed (a replay
 *    keeps the tag of its capture and still waits for its own partials).
 *    While one call enqueues its kernels it holds a host lock on its slot, so
 *    host threads that share a stream are safe.  A device on which more than
 *    64 streams have run reducing calls returns FP8Q_EUNSUPPORTED.
 *  - FP8Q_DEBUG set in the environment (to anything but "" or "0") makes every
 *    call print one line to stderr: the entry point, its integer arguments,
 *    the stream, the scratch slot and the returned status and message.  The
 *    line is printed after the kernels are enqueued and never waits for the
 *    device.
 *  - Enum-valued arguments are passed as int32_t (values below).
 *  - Tensors are dense and row-major.  FP8 tensors are arrays of 8-bit codes
 *    (uint8_t).  bf16 tensors are arrays of 16-bit bf16 patterns.
 *  - Element buffers (x, q, y, C) must be 16-byte aligned; scalar and scale
 *    buffers 4-byte aligned.
 *  - Errors: arguments are validated on the host before any HIP call.  A
 *    non-zero status is returned and a message is kept for
 *    fp8q_last_error() (thread-local).  Nothing is written on error.  A
 *    launch failure reported by the runtime returns FP8Q_EHIP, as does a
 *    valid call made where no device is usable (the message says why).
 *  - Numerics: scales, amaxes and the scaled values are binary32 with
 *    round-to-nearest-even.  The FP8 cast saturates to +-FP8_MAX and rounds to
 *    nearest, ties to even.  NaN is kept: a NaN product x*scale becomes code
 *    0x7F with the sign bit set to sign(x) XOR sign(scale).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FP8Q_OK 0
#define FP8Q_EINVAL 1      /* bad pointer, size, alignment or enum value */
#define FP8Q_EUNSUPPORTED 2 /* valid request the library does not implement */
#define FP8Q_EHIP 3        /* the HIP runtime reported an error */

/* FP8 formats, [MFP8] section 2.  E4M3FN: bias 7, max 448, no Inf, NaN only
 * S.1111.111.  E5M2: bias 15, max 57344, IEEE Inf and NaN. */
#define FP8Q_E4M3FN 0
#define FP8Q_E5M2 1

/* element types of high-precision tensors */
#define FP8Q_F32 0
#define FP8Q_BF16 1

/* delayed-scaling history reduction, [MFP8] section 5 */
#define FP8Q_ALGO_MAX 0
#define FP8Q_ALGO_MOST_RECENT 1

/* GEMM scaling modes */
#define FP8Q_PER_TENSOR 0
#define FP8Q_BLOCK_1x128_128x128 1
#define FP8Q_BLOCK_1x128_1x128 2
#define FP8Q_MXFP8 3

/* output types of fp8_scaled_gemm_fused beyond FP8Q_F32 / FP8Q_BF16: FP8
 * codes of the named format */
#define FP8Q_OUT_E4M3FN 2
#define FP8Q_OUT_E5M2 3

/* source of the columnwise copy in fp8_quantize_hybrid and
 * fp8_quantize_hybrid_blockwise, [HYBRID] */
#define FP8Q_COLSRC_ORIGINAL 0
#define FP8Q_COLSRC_ROWWISE_DEQUANTIZED 1

/* sub-quantizers of one direction in fp8_quantize_hybrid_blockwise, [HYBRID]
 * (the per-direction quantizer may be a blockwise, MXFP8 or per-tensor one) */
#define FP8Q_SUBQ_BLOCK_128x128 0 /* fp32 scale per 128x128 block, as fp8_quantize_block(block_rows 128) */
#define FP8Q_SUBQ_BLOCK_1x128 1   /* fp32 scale per 1x128 segment, as fp8_quantize_block(block_rows 1) */
#define FP8Q_SUBQ_MXFP8 2         /* E8M0 byte per 1x32 segment, as fp8_quantize_mx */
#define FP8Q_SUBQ_PER_TENSOR 3    /* one scale for the whole copy, as fp8_quantize_tensor */

/* epilogue activations, [MFP8] section 6 */
#define FP8Q_ACT_NONE 0
#define FP8Q_ACT_RELU 1
#define FP8Q_ACT_GELU 2

/*
 * fp8_amax -- *amax = max_i |x_i| over n elements ([MFP8] section 4, the
 * amax of compute_fp8_scale; section 11, tensor_amax).
 *   x      [n] elements of type `dtype` (FP8Q_F32 or FP8Q_BF16)
 *   amax   one float, written (overwritten) by the call
 * A NaN element gives the canonical NaN 0x7FC00000; n == 0 gives 0.
 * The result is exact (an integer max over magnitude bits, order-free).
 * Cache use: the call streams x, except its last 128 MiB, which it reads
 * with ordinary loads so that the cast of current scaling, which reads x
 * again right after it, finds them in the last-level cache.
 */
int fp8_amax(const void *x, int32_t dtype, int64_t n, float *amax, void *stream);

/*
 * fp8_quantize_tensor -- per-tensor scaled cast to FP8 ([MFP8] section 4
 * current scaling; section 5 delayed scaling, which consumes a stored scale).
 * Exactly one of amax_in / scale_inv_in is non-NULL:
 *   amax_in      (current scaling) s = fl32(max(*amax_in, 1e-12) / FP8_MAX) * 2^margin
 *   scale_inv_in (given scale)     s = *scale_inv_in, margin ignored
 * then scale = fl32(1 / s) and q_i = encode(fl32(x_i * scale)).
 *   x              [n] of `dtype`
 *   q              [n] FP8 codes of format `fmt`
 *   scale_inv_out  (nullable) receives s, the dequantization multiplier
 *   scale_out      (nullable) receives scale, the quantization multiplier
 *   amax_out       (nullable) receives max_i |x_i| of this input (fused, for
 *                  delayed scaling's history), defined as in fp8_amax
 * Output buffers must not overlap the inputs.
 */
int fp8_quantize_tensor(const void *x, int32_t dtype, int64_t n, int32_t fmt, const float *amax_in,
                        int32_t margin, const float *scale_inv_in, uint8_t *q, float *scale_inv_out,
                        float *scale_out, float *amax_out, void *stream);

/*
 * fp8_quantize_tensor_stats -- fp8_quantize_tensor that also counts, in the
 * same pass over x, what the cast did ([MFP8] section 24: per-tensor
 * overflow and underflow counts reported next to amax and scale; the counts
 * of fp8_cast_stats, taken against the scale s this call casts with, so that
 * monitoring a cast costs no second read of x):
 *   stats[0] overflows (x not NaN and |fl32(x * fl32(1/s))| > FP8_MAX),
 *   stats[1] underflows (x finite and nonzero with a zero code),
 *   stats[2] NaNs, stats[3] nonzeros (x not NaN and x != 0).
 *   stats  device uint64_t[4], 8-byte aligned, required; overwritten.
 * Every other argument, and every error, as in fp8_quantize_tensor; plus
 * FP8Q_EINVAL when stats is null, misaligned, or overlaps x, q or a scalar.
 */
int fp8_quantize_tensor_stats(const void *x, int32_t dtype, int64_t n, int32_t fmt, const float *amax_in,
                              int32_t margin, const float *scale_inv_in, uint8_t *q, float *scale_inv_out,
                              float *scale_out, float *amax_out, uint64_t *stats, void *stream);

/*
 * fp8_dequantize -- y_i = fl32(value(q_i) * *scale_inv) ([MFP8] section 4: the
 * cached inverse makes dequantization one element multiply; section 23:
 * reconstruction = fp8 value times scale).  With scale_inv = 1 over the 256
 * codes this is the decode table of the format.  NaN codes give a NaN
 * (payload unspecified); E5M2 Inf codes give +-Inf.
 *   q [n] codes, y [n] float32 output.
 */
int fp8_dequantize(const uint8_t *q, int32_t fmt, int64_t n, const float *scale_inv, float *y, void *stream);

/*
 * fp8_quantize_rowwise_colwise -- one per-tensor scale, two layouts ([HYBRID]:
 * a quantized tensor holds rowwise and columnwise storage; the columnwise one
 * is quantized from the original input).  Scale selection as in
 * fp8_quantize_tensor.
 *   x      [rows][cols] of `dtype`; rows and cols multiples of 16
 *   q_row  (nullable) [rows][cols] codes
 *   q_col  (nullable) [cols][rows] codes, q_col[j][i] = q_row[i][j]
 *   scale_inv_out, scale_out, amax_out (nullable) as in fp8_quantize_tensor
 * At least one of q_row / q_col must be given.
 */
int fp8_quantize_rowwise_colwise(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt,
                                 const float *amax_in, int32_t margin, const float *scale_inv_in, uint8_t *q_row,
                                 uint8_t *q_col, float *scale_inv_out, float *scale_out, float *amax_out,
                                 void *stream);

/*
 * fp8_quantize_block -- block current scaling with FP32 block scales
 * ([VIME] "BF16 Training with FP8 Rollout": 128x128 weight blocks;
 * "FP8 Quick Start": blockwise recipe with FP32 scales).  Each block gets
 * s_b = fl32(max(amax_b, 1e-12) / FP8_MAX) (margin 0), scale_b = fl32(1/s_b),
 * and its elements are cast with scale_b.  The stored scales are the s_b
 * (dequantization multipliers).
 *   x           [rows][cols] of `dtype`; rows, cols multiples of 128
 *   block_rows  128: 128x128 blocks.  1: 1x128 blocks (one row, 128 columns).
 *   q_row [rows][cols] codes, s_row [rows/block_rows][cols/128]
 *   q_col, s_col (nullable, both or neither): the columnwise copy, i.e. the
 *     same rule applied to x^T: q_col [cols][rows].
 *     128x128: q_col = q_row^T, s_col [cols/128][rows/128] = s_row^T.
 *     1x128:   blocks of 128 consecutive rows of one column of x,
 *              s_col [cols][rows/128].
 */
int fp8_quantize_block(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt, int32_t block_rows,
                       uint8_t *q_row, float *s_row, uint8_t *q_col, float *s_col, void *stream);

/*
 * fp8_quantize_mx -- MXFP8 quantization ([MFP8] section 16: 32 consecutive
 * elements share one E8M0 scale, 8 exponent bits, no mantissa or sign,
 * 2^-127 .. 2^127; section 10: the finest-grained recipe).  The pages leave
 * the choice of the shared exponent open; this library takes the OCP
 * Microscaling rule: for a block with magnitude max a,
 *   e = floor(log2(a)) - emax (emax = 8 for E4M3FN, 15 for E5M2), clamped to
 *   [-127, 127]; an all-zero block takes e = -127, an infinite a e = 127;
 *   the scale byte is e + 127 (255, NaN, when the block holds a NaN) and each
 *   element is encoded from fl32(x * 2^-e) like every other cast (saturating,
 *   round to nearest even; a NaN block's elements become NaN codes).
 *   x      [rows][cols] of `dtype`; rows, cols multiples of 128
 *   q_row  [rows][cols] codes; s_row [rows][cols/32] scale bytes (blocks of 32
 *          consecutive columns of a row: the K-contiguous operand of the
 *          FP8Q_MXFP8 GEMM)
 *   q_col, s_col (nullable, both or neither): the columnwise copy, the same
 *          rule applied to x^T: q_col [cols][rows], s_col [cols][rows/32].
 *   Code buffers 16-byte aligned, scale buffers 4-byte aligned.
 */
int fp8_quantize_mx(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt, uint8_t *q_row,
                    uint8_t *s_row, uint8_t *q_col, uint8_t *s_col, void *stream);

/*
 * fp8_update_scale_delayed -- delayed-scaling state update ([MFP8] section 5,
 * the amax-history ring and the fp8_meta update).
 *   hist       [history_len][n_cols] float history, column `col` is updated
 *   new_amax   one float (device), the amax measured by the step just run
 *   step       host count of earlier updates of this column; the value is
 *              written at slot step % history_len
 *   fmt        format whose FP8_MAX the new scale targets (the format of the
 *              tensor that will consume it)
 *   algo       FP8Q_ALGO_MAX: eff = max of the column's history (NaN if any
 *              NaN); FP8Q_ALGO_MOST_RECENT: eff = *new_amax
 *   scale, scale_inv  [n_cols]; entry `col` receives
 *              s = eff > 0 ? fl32(eff / FP8_MAX) * 2^margin : 1  (scale_inv)
 *              and fl32(1 / s) (scale)
 * The initial state of a column is hist = 0, scale = scale_inv = 1.
 */
int fp8_update_scale_delayed(float *hist, int32_t history_len, int32_t n_cols, int32_t col, const float *new_amax,
                             int64_t step, int32_t fmt, int32_t margin, int32_t algo, float *scale, float *scale_inv,
                             void *stream);

/*
 * fp8_quantize_delayed -- one delayed-scaling step ([MFP8] section 5: cast
 * with the scale derived from the history, then record this input's amax and
 * derive the scale for the next step).  Equivalent to
 *   fp8_quantize_tensor(x, dtype, n, fmt, NULL, 0, &scale_inv[col], q,
 *                       q_scale_inv_out, NULL, amax_out', stream)
 *   fp8_update_scale_delayed(hist, history_len, n_cols, col, amax_out', step,
 *                            fmt_next, margin, algo, scale, scale_inv, stream)
 * with the amax handed from the cast to the update on the device (two kernel
 * launches instead of three).
 *   x, dtype, n, fmt   the tensor of this step and its FP8 format
 *   hist, history_len, n_cols, col, step, margin, algo, scale, scale_inv
 *                      the delayed-scaling state, as in fp8_update_scale_delayed
 *   fmt_next           format whose FP8_MAX the new scale targets
 *   q                  [n] codes
 *   q_scale_inv_out    (nullable) receives the s this step was cast with
 *   amax_out           (nullable) receives max |x|
 * Errors: the checks of both calls above, plus FP8Q_EINVAL when x or q
 * overlaps hist, scale, scale_inv or a scalar output.
 */
int fp8_quantize_delayed(const void *x, int32_t dtype, int64_t n, int32_t fmt, float *hist, int32_t history_len,
                         int32_t n_cols, int32_t col, int64_t step, int32_t fmt_next, int32_t margin, int32_t algo,
                         float *scale, float *scale_inv, uint8_t *q, float *q_scale_inv_out, float *amax_out,
                         void *stream);

/*
 * fp8_scaled_gemm -- C = (A * sA) (B * sB)^T on FP8 codes with fp32
 * accumulation ([MFP8] section 6: FP8 operands and fp32 accumulation, bf16
 * output for fprop and dgrad, fp32 output for wgrad = dY^T X; section 27:
 * products promoted to fp32 and summed, one downcast of the finished dot
 * product).
 *   A [M][K] codes of format fa, B [N][K] codes of format fb (both
 *   K-contiguous), C [M][N] output of type c_dtype (FP8Q_BF16 or FP8Q_F32).
 *   mode FP8Q_PER_TENSOR: sA, sB point to one float each (dequant scales);
 *        C = out(fl32(fl32(sA*sB) * acc)).
 *   mode FP8Q_BLOCK_1x128_128x128: sA [M][K/128] (1x128 blocks of A),
 *        sB [N/128][K/128] (128x128 blocks of B); each 128-wide K slice is
 *        accumulated separately and added as
 *        acc = fma(part, fl32(sA[m,kb]*sB[n/128,kb]), acc); C = out(acc).
 *   mode FP8Q_BLOCK_1x128_1x128: as above with sB [N][K/128] (1x128 blocks
 *        of B, one scale per row of B and K slice), the weight gradient from
 *        the transposed (token-contiguous) copies of dY and X.
 *   mode FP8Q_MXFP8 ([MFP8] sections 10 and 16): sA [M][K/32] and sB
 *        [N][K/32] are E8M0 scale bytes (const uint8_t data passed through the
 *        float pointers), one per 32-element block along K; every element is
 *        multiplied by 2^(byte - 127) of its block (by the matrix instruction
 *        itself) and C = out(acc).
 *   out() is bf16 round-to-nearest-even or the fp32 value itself.
 *   amax_out (nullable) receives max |C| over the emitted values.
 * M, N, K must be multiples of 128, K at most 2^22 and M, N at most 2^31
 * (FP8Q_EUNSUPPORTED otherwise).
 */
int fp8_scaled_gemm(const uint8_t *A, int32_t fa, const float *sA, const uint8_t *B, int32_t fb, const float *sB,
                    int64_t M, int64_t N, int64_t K, int32_t mode, void *C, int32_t c_dtype, float *amax_out,
                    void *stream);

/*
 * fp8_scaled_gemm_fused -- fp8_scaled_gemm with the epilogue fusions of
 * [MFP8] section 6 (bias addition and an activation folded into the GEMM
 * epilogue, so the intermediate never makes a bf16 round trip through
 * memory) and an FP8 output cast with a given scale, whose amax feeds the
 * next scaling decision ([MFP8] section 4: amax of the high-precision tensor
 * recorded for delayed scaling; section 5: the history update).
 *   A, fa, sA, B, fb, sB, M, N, K, mode: as fp8_scaled_gemm; v[m,n] is the
 *   value fp8_scaled_gemm would round to its output type (fp32).
 *   bias (nullable): fp32 [N], 16-byte aligned; added along the rows:
 *        y = act(v[m,n] + bias[n]) in binary32.
 *   act: FP8Q_ACT_NONE; FP8Q_ACT_RELU (y < 0 -> 0, NaN kept);
 *        FP8Q_ACT_GELU, the exact form v * Phi(v), Phi the standard normal
 *        CDF (not the tanh approximation), evaluated in binary32 to within
 *        2^-21 |v| of v * Phi(v); +inf maps to +inf, -inf and NaN to NaN.
 *   C [M][N] of type c_type: FP8Q_BF16 (round to nearest even), FP8Q_F32, or
 *        FP8Q_OUT_E4M3FN / FP8Q_OUT_E5M2: codes of fl32(y * fl32(1/s)) with
 *        s = *c_scale_inv (the output's dequant scale, 4-byte aligned float,
 *        required for and only for FP8 outputs), saturating RNE cast.
 *   amax_out (nullable): max |C| over the emitted values for bf16 / fp32
 *        output, max |y| over the values before the cast for FP8 output.
 * Errors: those of fp8_scaled_gemm; FP8Q_EINVAL for an unknown c_type or
 * act, a missing or stray c_scale_inv, a misaligned bias, or C or amax_out
 * overlapping bias or c_scale_inv.
 */
int fp8_scaled_gemm_fused(const uint8_t *A, int32_t fa, const float *sA, const uint8_t *B, int32_t fb,
                          const float *sB, int64_t M, int64_t N, int64_t K, int32_t mode, const float *bias,
                          int32_t act, void *C, int32_t c_type, const float *c_scale_inv, float *amax_out,
                          void *stream);

/*
 * fp8_quantize_hybrid -- per-direction ("hybrid") per-tensor quantization of
 * a 2-D tensor ([HYBRID]: the rowwise and the columnwise copies may use
 * different formats and scaling recipes; the columnwise copy is quantized
 * from the original input or from the dequantized rowwise values).
 *   x [rows][cols] of dtype; q_row [rows][cols] codes of row_fmt,
 *   q_col [cols][rows] codes of col_fmt (either may be NULL, not both unless
 *   the tensor is empty; with the dequantized source the row codes are formed
 *   even when q_row is NULL).  An empty tensor still publishes both scales
 *   and an amax of 0.
 *   col_source FP8Q_COLSRC_ORIGINAL: q_col = cast of x^T;
 *              FP8Q_COLSRC_ROWWISE_DEQUANTIZED: q_col = cast of x'^T with
 *              x' = fl32(value(q_row) * s_row).
 *   Scales, exactly one way:
 *     amax_in (= max |x|): current scaling per direction of its own source,
 *       s_row from amax_in with row_fmt and row_margin; s_col from amax_in
 *       (original source) or from max |x'| (which the cast maps exactly from
 *       amax_in, so no second pass) with col_fmt and col_margin;
 *     row_scale_inv_in and col_scale_inv_in: the two given dequant scales
 *       (delayed scaling, one history per direction).
 *   Each direction casts with fl32(1/s) like fp8_quantize_tensor.
 *   row_scale_inv_out, col_scale_inv_out, amax_out (nullable): the scales
 *   used and max |x| (fused).
 * rows, cols: multiples of 16 (FP8Q_EUNSUPPORTED otherwise).
 * Errors: FP8Q_EINVAL for unknown enums, a wrong combination of scale
 * inputs, misalignment, or overlapping buffers (scalar outputs may not alias
 * inputs or each other).
 */
int fp8_quantize_hybrid(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t row_fmt, int32_t col_fmt,
                        int32_t col_source, const float *amax_in, int32_t row_margin, int32_t col_margin,
                        const float *row_scale_inv_in, const float *col_scale_inv_in, uint8_t *q_row, uint8_t *q_col,
                        float *row_scale_inv_out, float *col_scale_inv_out, float *amax_out, void *stream);

/*
 * fp8_quantize_hybrid_blockwise -- per-direction ("hybrid") quantization with
 * block sub-quantizers ([HYBRID]: each direction has a quantizer of its own,
 * with its own format and recipe, blockwise and MXFP8 ones included; the
 * columnwise copy is quantized from the original input or from the
 * dequantized rowwise values).
 *   x [rows][cols] of dtype; rows, cols multiples of 128.
 *   Rowwise copy: row_recipe in row_fmt applied to x, exactly what
 *     fp8_quantize_block / fp8_quantize_mx write as q_row and s_row:
 *     q_row [rows][cols]; s_row float [rows/128][cols/128] (128x128),
 *     float [rows][cols/128] (1x128) or E8M0 bytes [rows][cols/32] (MXFP8).
 *   Columnwise copy: col_recipe in col_fmt applied to y^T, what those calls
 *     write as q_col and s_col: q_col [cols][rows]; s_col float
 *     [cols/128][rows/128], float [cols][rows/128] or bytes [cols][rows/32].
 *     col_source FP8Q_COLSRC_ORIGINAL: y = x;
 *     FP8Q_COLSRC_ROWWISE_DEQUANTIZED: y = x' = fl32(value(q_row) * d)
 *     elementwise, d the dequant scale of the element's row block (the FP32
 *     block scale, or 2^(byte - 127) for MXFP8, NaN for byte 255); where x'
 *     is NaN (a NaN row code, or a zero code times an infinite block scale)
 *     its column code is the NaN code with the row code's sign bit.  The row
 *     codes are formed even when q_row is NULL.
 *   FP8Q_SUBQ_PER_TENSOR in one direction (not both: two per-tensor
 *     directions are fp8_quantize_hybrid's): that copy is the per-tensor cast
 *     of fp8_quantize_tensor with the scale from amax_in (current scaling,
 *     with margin) or from scale_inv_in (exactly one of them, device floats);
 *     its scale buffer is one float that receives the dequant scale s used
 *     (the dequantized rows of a per-tensor row copy use that s).  Per-tensor
 *     columns of the dequantized rows take scale_inv_in only (their amax is
 *     not known before the pass: FP8Q_EUNSUPPORTED with amax_in).  Without a
 *     per-tensor direction amax_in and scale_inv_in must be NULL.
 *   Either copy may be skipped (its code and scale pointers both NULL), not
 *   both.  The call reads x once, whatever the two recipes and formats (with
 *   one recipe both ways, both formats take their scales from the same block
 *   maxima).  Scale pointers are void *: float or byte buffers as above,
 *   4-byte aligned; code buffers 16-byte aligned.
 * Errors: FP8Q_EINVAL for unknown enums, a code pointer without its scale
 * pointer (or the reverse), no copy at all, two per-tensor directions, a
 * per-tensor direction without exactly one of amax_in / scale_inv_in (or
 * either of them without a per-tensor direction), misalignment or overlapping
 * buffers; FP8Q_EUNSUPPORTED for shapes that are not multiples of 128 and for
 * per-tensor columns of the dequantized rows with amax_in.
 */
int fp8_quantize_hybrid_blockwise(const void *x, int32_t dtype, int64_t rows, int64_t cols, int32_t row_recipe,
                                  int32_t row_fmt, uint8_t *q_row, void *s_row, int32_t col_recipe, int32_t col_fmt,
                                  int32_t col_source, uint8_t *q_col, void *s_col, const float *amax_in,
                                  int32_t margin, const float *scale_inv_in, void *stream);

/*
 * fp8_cast_stats -- diagnostics of the per-tensor cast of x with dequant
 * scale *scale_inv ([MFP8] section 24: per-tensor overflow and underflow
 * counts reported next to amax and scale).  With y = fl32(x * fl32(1/s)):
 *   stats[0] overflows:  x not NaN and |y| > FP8_MAX (saturated by the cast);
 *   stats[1] underflows: x finite and nonzero whose code is a zero code;
 *   stats[2] NaNs;  stats[3] nonzeros (x not NaN and x != 0).
 * stats: device uint64_t[4], 8-byte aligned.  x is read once (no codes are
 * written).
 */
int fp8_cast_stats(const void *x, int32_t dtype, int64_t n, int32_t fmt, const float *scale_inv, uint64_t *stats,
                   void *stream);

/*
 * fp8_quantize_error_feedback -- one step of FP8 quantization with error
 * feedback ([MFP8] section 25: quantize g plus the carried residual, keep what
 * the cast lost for the next step, so the sum of what is sent tracks the sum
 * of the inputs):
 *   v = fl32(g + residual);  q = codes of fl32(v * fl32(1/s)), s = *scale_inv;
 *   residual <- fl32(v - fl32(value(q) * s))   (in place);
 *   amax_out (nullable) <- max |v| (for the next delayed-scaling update).
 * g: n elements of dtype; residual: fp32 [n], 16-byte aligned, read and
 * written; q: n codes of fmt.
 */
int fp8_quantize_error_feedback(const void *g, int32_t dtype, float *residual, int64_t n, int32_t fmt,
                                const float *scale_inv, uint8_t *q, float *amax_out, void *stream);

/*
 * fp8q_clock_monitor -- a measurement aid, not a step of the method: the
 * graphics clock that other work runs at.  Enqueues on `stream` one kernel of
 * 8 one-wave blocks (consecutive blocks start on consecutive XCDs; each needs
 * only a few registers, so it shares a CU with the work being measured).
 * Each block counts its CU's shader-clock cycles and the chip's constant-rate
 * ticks from its start until *stop is nonzero, or 2 seconds of the constant
 * counter, whichever comes first.  cycles / (ticks / rate) is the CU's average
 * clock over that interval.  Use: zero *stop, enqueue this on a side stream,
 * enqueue the work on another stream, then make *stop nonzero from a kernel
 * on the work's stream (the blocks read it with agent-scope loads) and
 * synchronize.
 * out: device uint64[25], 8-byte aligned, written when the kernel ends:
 *   out[3 b + 0] XCD id of block b (b = 0..7), out[3 b + 1] shader-clock
 *   cycles, out[3 b + 2] constant-rate ticks, out[24] the constant rate in
 *   kHz.
 * stop: device uint32, 4-byte aligned, read only.
 * Errors: FP8Q_EINVAL for a null, misaligned or overlapping pointer;
 * FP8Q_EHIP from the launch.  Uses no scratch.
 */
int fp8q_clock_monitor(uint64_t *out, const uint32_t *stop, void *stream);

/*
 * fp8q_set_finish_poll_rounds -- a failure-handling knob, not a step of the
 * method.  A reducing call whose launch ends in a finishing block (fp8_amax,
 * the casts with amax_out, fp8_quantize_delayed) has that block wait for the
 * other blocks' partials for at most `rounds` polling rounds (default
 * 2^21, about a second and more); past the bound the call's amax is the
 * canonical NaN (and fp8_quantize_delayed records NaN in its ring).  Partials
 * that arrive after the bound carry that call's tag and are ignored by every
 * later eager call (a graph replay reuses its capture's tag, so a replay
 * after one that gave up could take such a late partial).  rounds = 0 makes every finishing block give up at once (used
 * by the tests of this path); 0xFFFFFFFF restores the default.  Applies to
 * calls made afterwards, in every thread, on every device.
 * previous: host uint32 or NULL; receives the bound that was in force.
 * Returns FP8Q_OK.  Enqueues nothing.
 */
int fp8q_set_finish_poll_rounds(uint32_t rounds, uint32_t *previous);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char *fp8q_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
