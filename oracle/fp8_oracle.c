/*
 * fp8_oracle.c -- plain CPU oracle for FP8 scaled quantization and the scaled
 * FP8 GEMM's scalar parts.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source, header, table or constant generator
 * with the HIP library; it is written from the definitions on the reference
 * pages, in the order those pages state them, without blocking or fusion.
 *
 * Pages cited (title, section):
 *   [MFP8]   "Megatron FP8"  (sections numbered 1-28 on that page)
 *   [HYBRID] "[Pytorch][Common] Hybrid quantization #2817" (TransformerEngine PR)
 *   [VIME]   "Low Precision Training and Rollout" (vime documentation)
 *
 * Floating point: the pages keep scales, amaxes and the scaled tensor in FP32
 * ([MFP8] section 4 code and section 5 "state tensors (FP32)"), so the scalar
 * arithmetic below is binary32 with round-to-nearest-even, exactly as C on
 * x86-64 SSE evaluates `float` expressions (build with -ffp-contract=off).
 * Decoded FP8 values and distances between them are handled in binary64,
 * where they are exact.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_E4M3FN 0
#define ORC_E5M2 1
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_ALGO_MAX 0
#define ORC_ALGO_MOST_RECENT 1

/* ------------------------------------------------------------------------ */
/* Bit layouts.  [MFP8] section 2: E4M3 is 1 sign, 4 exponent, 3 mantissa bits;
 * E5M2 is 1 sign, 5 exponent, 2 mantissa bits; bias = 2^(k-1) - 1 for k
 * exponent bits. */
static int exp_bits(int fmt) { return fmt == ORC_E4M3FN ? 4 : 5; }
static int man_bits(int fmt) { return fmt == ORC_E4M3FN ? 3 : 2; }
static int bias_of(int fmt) { return (1 << (exp_bits(fmt) - 1)) - 1; }

/* Decode one 8-bit code to its value.  [MFP8] section 2: normal numbers follow
 * the IEEE 754 rule; E5M2 keeps IEEE Inf (all-ones exponent, zero mantissa)
 * and NaN (all-ones exponent, nonzero mantissa); E4M3FN has no Inf and only
 * the all-ones exponent with all-ones mantissa is NaN, which leaves 448 as the
 * largest finite value.  Exponent field zero holds the subnormals, which fill
 * the gap between zero and the smallest normal ([MFP8] section 3). */
double orc_decode(int fmt, int code)
{
    const int mb = man_bits(fmt), eb = exp_bits(fmt), bias = bias_of(fmt);
    const int s = (code >> 7) & 1;
    const int e = (code >> mb) & ((1 << eb) - 1);
    const int m = code & ((1 << mb) - 1);
    const double sign = s ? -1.0 : 1.0;
    if (fmt == ORC_E4M3FN) {
        if (e == 15 && m == 7) return s ? -NAN : NAN;
    } else {
        if (e == 31) {
            if (m == 0) return sign * INFINITY;
            return s ? -NAN : NAN;
        }
    }
    if (e == 0) /* subnormal: m * 2^(1 - bias - mant_bits) */
        return sign * ldexp((double)m, 1 - bias - mb);
    return sign * ldexp(1.0 + (double)m / (double)(1 << mb), e - bias);
}

/* Largest non-negative finite code: 0x7E (448) for E4M3FN, 0x7B (57344) for
 * E5M2. */
int orc_max_code(int fmt) { return fmt == ORC_E4M3FN ? 0x7E : 0x7B; }

/* FP8_MAX of the format, as the value of its largest finite code. */
double orc_fmax(int fmt) { return orc_decode(fmt, orc_max_code(fmt)); }

/* Table of the non-negative finite values, index = code (0 .. max code).  The
 * codes are in increasing order of value, which the pin tests check. */
static double pos_table[2][128];

/* Filled once when the library is loaded, before any parallel loop runs. */
__attribute__((constructor)) static void fill_tables(void)
{
    for (int f = 0; f < 2; ++f)
        for (int c = 0; c <= orc_max_code(f); ++c) pos_table[f][c] = orc_decode(f, c);
}

static const double *values_of(int fmt) { return pos_table[fmt]; }

/* Encode one binary32 value y (already multiplied by the scale) to a code.
 *  - NaN keeps its sign and becomes the format's NaN code 0x7F / 0xFF.
 *  - Magnitudes above FP8_MAX, infinities included, are clipped to FP8_MAX:
 *    the clip-before-cast of [MFP8] section 4, and E4M3FN's "overflow
 *    saturates to +-448, never to Inf" of [MFP8] section 2, applied to both
 *    formats.
 *  - Otherwise the code whose value is nearest to |y|; on an exact tie the
 *    code with the even mantissa, i.e. the even code ([MFP8] section 23:
 *    round-to-nearest-even).
 *  - The sign bit is copied, so -0 and negative underflow give 0x80. */
uint8_t orc_encode(int fmt, float y)
{
    uint32_t bits;
    memcpy(&bits, &y, 4);
    const int sign = (int)(bits >> 31);
    if (isnan(y)) return (uint8_t)((sign << 7) | 0x7F);
    const double *v = values_of(fmt);
    const int top = orc_max_code(fmt);
    double a = fabs((double)y);
    if (a > v[top]) a = v[top];
    /* c = largest code with v[c] <= a (binary search over the ordered table) */
    int lo = 0, hi = top;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (v[mid] <= a) lo = mid;
        else hi = mid - 1;
    }
    int c = lo;
    if (c < top) {
        /* both differences are exact in binary64 */
        const double below = a - v[c], above = v[c + 1] - a;
        if (above < below || (above == below && (c & 1))) c = c + 1;
    }
    return (uint8_t)((sign << 7) | c);
}

/* Encode a buffer of binary32 values that are already scaled. */
void orc_encode_buffer(int fmt, const float *y, int64_t n, uint8_t *q)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) q[i] = orc_encode(fmt, y[i]);
}

/* bf16 -> binary32 is exact: the bf16 bits are the high half of the binary32 */
static float bf16_to_f32(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static float load_elem(const void *x, int dtype, int64_t i)
{
    if (dtype == ORC_F32) return ((const float *)x)[i];
    return bf16_to_f32(((const uint16_t *)x)[i]);
}

static float canonical_nan(void)
{
    uint32_t b = 0x7FC00000u;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* amax = max_i |x_i|.  [MFP8] section 4 (`x.abs().max()`) and section 11
 * (`tensor_amax`).  Any NaN element makes the result NaN (as the tensor max
 * does); it is returned as the canonical quiet NaN.  An empty tensor gives 0. */
float orc_amax(const void *x, int dtype, int64_t n)
{
    float m = 0.0f;
    int saw_nan = 0;
#pragma omp parallel for reduction(max : m) reduction(| : saw_nan) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(load_elem(x, dtype, i));
        if (isnan(a)) saw_nan = 1;
        else if (a > m) m = a;
    }
    return saw_nan ? canonical_nan() : m;
}

/* The amax floor of the current-scaling code, `clamp_min(1e-12)`
 * ([MFP8] section 4), as a binary32 constant. */
static const float AMAX_FLOOR = 1e-12f;

/* Current scaling, [MFP8] section 4 (compute_fp8_scale) and section 10
 * (margin): s* = amax / FP8_MAX with amax clamped below at 1e-12,
 * s = s* * 2^margin.  s is what the page calls the scaling factor; dequantizing
 * multiplies by it, so it is returned as scale_inv.  The quantizing
 * multiplier is its binary32 reciprocal, returned as scale ([MFP8] section 4:
 * the inverse is cached so that a rescale is one element multiply).
 * A NaN amax gives NaN for both. */
void orc_current_scale(float amax, int fmt, int margin, float *scale_inv, float *scale)
{
    const float fmax = (float)orc_fmax(fmt);
    float ac = isnan(amax) ? amax : (amax > AMAX_FLOOR ? amax : AMAX_FLOOR);
    float s_star = ac / fmax;
    float s = ldexpf(s_star, margin);
    *scale_inv = s;
    *scale = 1.0f / s;
}

/* Code of one scaled element, [MFP8] section 4: the element is multiplied by
 * the quantizing scale in binary32 and the product is encoded (saturation and
 * round-to-nearest-even inside orc_encode).  IEEE 754 leaves the sign of a NaN
 * produced by an invalid product (Inf * 0) unspecified, and hardware differs,
 * so a NaN product takes the sign rule of multiplication: sign(x) XOR
 * sign(scale).  For a NaN x and a positive scale that is x's own sign. */
static uint8_t encode_product(int fmt, float x, float scale)
{
    float y = x * scale;
    if (isnan(y)) {
        int sx = signbit(x) ? 1 : 0, ss = signbit(scale) ? 1 : 0;
        return (uint8_t)(((sx ^ ss) << 7) | 0x7F);
    }
    return orc_encode(fmt, y);
}

/* Per-tensor cast: every element with the same quantizing scale. */
void orc_quantize(const void *x, int dtype, int64_t n, int fmt, float scale, uint8_t *q)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) q[i] = encode_product(fmt, load_elem(x, dtype, i), scale);
}

/* Dequantize: value of the code times scale_inv, rounded to binary32
 * ([MFP8] section 4: dequantization is one element multiply by the cached
 * inverse; section 23: reconstructed = fp8 value * scale). */
void orc_dequantize(const uint8_t *q, int fmt, int64_t n, float scale_inv, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float v = (float)orc_decode(fmt, q[i]); /* exact: every code fits binary32 */
        y[i] = v * scale_inv;
    }
}

/* Rowwise + columnwise copy with one per-tensor scale ([HYBRID]: a quantized
 * tensor carries rowwise storage and columnwise storage, the columnwise one
 * quantized from the original input by default).  q_row is [rows][cols];
 * q_col is [cols][rows] and holds the code of x[i][j] at (j, i). */
void orc_quantize_rowwise_colwise(const void *x, int dtype, int64_t rows, int64_t cols, int fmt,
                                  float scale, uint8_t *q_row, uint8_t *q_col)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) {
            uint8_t c = encode_product(fmt, load_elem(x, dtype, i * cols + j), scale);
            if (q_row) q_row[i * cols + j] = c;
            if (q_col) q_col[j * rows + i] = c;
        }
}

/* Block scaling ([VIME] "BF16 Training with FP8 Rollout": weights quantized in
 * 128x128 blocks; "FP8 Quick Start": blockwise recipe with FP32 block scales).
 * Each block gets current scaling with margin 0 from its own amax, and its
 * elements are cast with that block's scale.  Blocks of br rows x bc columns
 * tile x [rows][cols] exactly.  s_out[I][J] = the block's dequant scale
 * (scale_inv), laid out [rows/br][cols/bc]. */
void orc_quantize_block(const void *x, int dtype, int64_t rows, int64_t cols, int fmt,
                        int64_t br, int64_t bc, uint8_t *q, float *s_out)
{
    const int64_t nbr = rows / br, nbc = cols / bc;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t I = 0; I < nbr; ++I)
        for (int64_t J = 0; J < nbc; ++J) {
            float m = 0.0f;
            int saw_nan = 0;
            for (int64_t i = I * br; i < (I + 1) * br; ++i)
                for (int64_t j = J * bc; j < (J + 1) * bc; ++j) {
                    float a = fabsf(load_elem(x, dtype, i * cols + j));
                    if (isnan(a)) saw_nan = 1;
                    else if (a > m) m = a;
                }
            float amax = saw_nan ? canonical_nan() : m;
            float s, sc;
            orc_current_scale(amax, fmt, 0, &s, &sc);
            s_out[I * nbc + J] = s;
            for (int64_t i = I * br; i < (I + 1) * br; ++i)
                for (int64_t j = J * bc; j < (J + 1) * bc; ++j)
                    q[i * cols + j] = encode_product(fmt, load_elem(x, dtype, i * cols + j), sc);
        }
}

/* Transpose of a [rows][cols] matrix of `es`-byte elements into [cols][rows].
 * Used to build the columnwise block copies: the columnwise copy is the same
 * rule applied to the transposed input. */
void orc_transpose(const void *x, int64_t rows, int64_t cols, int64_t es, void *xt)
{
    const char *src = (const char *)x;
    char *dst = (char *)xt;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) memcpy(dst + (j * rows + i) * es, src + (i * cols + j) * es, (size_t)es);
}

/* Delayed scaling update, [MFP8] section 5 (AmaxHistory ring and the
 * fp8_meta update): the newly measured amax goes to slot step % history_len of
 * column `col` of hist [history_len][n_cols]; the effective amax is the
 * maximum over the column's whole history (algo "max") or the value just
 * written ("most_recent"); the new scaling factor is
 * eff / FP8_MAX * 2^margin when eff > 0, else 1 (the ring class's rule for an
 * empty history).  scale_inv[col] receives that factor, scale[col] its
 * binary32 reciprocal.  A NaN in the history makes eff NaN, hence not > 0. */
void orc_delayed_update(float *hist, int history_len, int n_cols, int col, float new_amax, int64_t step,
                        int fmt, int margin, int algo, float *scale, float *scale_inv)
{
    const int64_t slot = step % history_len;
    hist[slot * n_cols + col] = new_amax;
    float eff;
    if (algo == ORC_ALGO_MAX) {
        int saw_nan = 0;
        eff = -INFINITY;
        for (int j = 0; j < history_len; ++j) {
            float h = hist[(int64_t)j * n_cols + col];
            if (isnan(h)) saw_nan = 1;
            else if (h > eff) eff = h;
        }
        if (saw_nan) eff = canonical_nan();
    } else {
        eff = new_amax;
    }
    const float fmax = (float)orc_fmax(fmt);
    float s = (eff > 0.0f) ? ldexpf(eff / fmax, margin) : 1.0f;
    scale_inv[col] = s;
    scale[col] = 1.0f / s;
}

/* MXFP8 ([MFP8] sections 10 and 16; the OCP Microscaling format the pages
 * name): every 32 consecutive elements of a row share one E8M0 scale, a
 * power of two 2^(b - 127) stored as the byte b (0..254; 255 is NaN), and each
 * element is an E4M3FN or E5M2 code.  The pages do not spell out how the
 * shared exponent is chosen; the reading here is the OCP rule: the largest
 * power of two not above the block's amax, divided by the format's largest
 * power of two (2^8 for E4M3FN, 2^15 for E5M2), so that the block's largest
 * element lands in the format's top binade:
 *   e = floor(log2(amax)) - emax, clamped to [-127, 127]; b = e + 127;
 *   q = encode(fl32(x * 2^-e)).
 * An all-zero block takes e = -127.  A NaN amax gives b = 255 and NaN codes
 * (x times NaN).  An infinite amax clamps e to 127. */
void orc_quantize_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t *q, uint8_t *scales)
{
    const int emax = fmt == ORC_E4M3FN ? 8 : 15;
    const int64_t nblk = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t bj = 0; bj < nblk; ++bj) {
            const int64_t j0 = bj * 32;
            float a = 0.0f;
            int saw_nan = 0;
            for (int64_t j = j0; j < j0 + 32; ++j) {
                const float v = load_elem(x, dtype, i * cols + j);
                if (isnan(v)) saw_nan = 1;
                else if (fabsf(v) > a) a = fabsf(v);
            }
            int e;
            float mult;
            if (saw_nan) {
                scales[i * nblk + bj] = 255;
                mult = canonical_nan();
            } else {
                if (a == 0.0f) e = -127;
                else if (isinf(a)) e = 127;
                else {
                    e = ilogbf(a) - emax; /* floor(log2(a)), subnormal a included */
                    if (e < -127) e = -127;
                    if (e > 127) e = 127;
                }
                scales[i * nblk + bj] = (uint8_t)(e + 127);
                mult = ldexpf(1.0f, -e); /* exact: 2^-127 .. 2^127 */
            }
            for (int64_t j = j0; j < j0 + 32; ++j)
                q[i * cols + j] = encode_product(fmt, load_elem(x, dtype, i * cols + j), mult);
        }
    }
}

/* Decode a whole code buffer to binary64 (the GEMM reference's operands). */
void orc_decode_buffer(const uint8_t *q, int fmt, int64_t n, double *out)
{
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = orc_decode(fmt, c);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = table[q[i]];
}

/* Number of OpenMP threads the parallel loops above use. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
