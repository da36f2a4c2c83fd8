/*
 * lowbit_oracle.c -- CPU oracle for the low-bit weight-only matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  This file states, as plainly as possible and in
 * double precision, what the GPU library computes.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant with the GPU library, and the GPU library
 * never calls it.
 *
 * Rules followed here: single thread, no SIMD intrinsics, no fast-math, plain
 * loops in the order the definitions are written, every floating-point
 * quantity carried in IEEE double (binary64) unless a step is defined in a
 * narrower type.
 *
 * Sources (web pages, cited by title and section):
 *   [Metal]  "Low Bit Metal Kernels" (GPU MODE lecture 49 notes), the MSL
 *            listing `int4_matmul`, step 2 (INT4 dequant) and step 3 (tile
 *            matmul).
 *   [ARM]    "Low Bit ARM kernels" (GPU MODE lecture 38 notes), section on
 *            group-wise quantization (symmetric / asymmetric, fp16 scale plus
 *            int8 zero point per group, group sizes 32/64/128), the section
 *            on decode = GEMV, prefill = GEMM, and the measurements section
 *            (4-bit weights with dynamic INT8 activations, group 32).
 *   [LUT-B]  "vLLM PR #62759 analysis: decoding LUT-B MoE weights directly in
 *            Rubin tensor cores with MXFP8 activations", sections "Format"
 *            (3-bit index, E4M3 codebook per 8 output channels x 64 K, one
 *            UE8M0 exponent per tile), "A gather" (sorted_token_ids,
 *            row_valid), "Expert parallelism" (non-local expert -> zero rows)
 *            and "Emulation path" (dequantize weights, MXFP8 q->dq of
 *            activations, BF16 expert GEMM).
 *
 * Every function's readings of points the pages leave open are listed in the
 * comment above it.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>

/* ------------------------------------------------------------------------ */
/* Number formats, from the IEEE 754 / OCP MX definitions.                  */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* f/128 * 2^-126 */
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/128) * 2^(e-127) */
    return sign ? -v : v;
}

/* Round-to-nearest-even of an integer-valued scaling: returns the integer
 * nearest to t >= 0, ties to even.  t is exact (a double scaled by a power of
 * two), so floor and the comparison are exact. */
static double rne_nonneg(double t)
{
    double fl = floor(t);
    double r = t - fl;
    if (r > 0.5) return fl + 1.0;
    if (r < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Generic RNE of |v| onto a binary format with `p` significand bits
 * (including the hidden bit), minimum normal exponent emin and maximum
 * finite value vmax.  Returns the rounded magnitude, INFINITY on overflow. */
static double round_to_format(double a, int p, int emin, double vmax)
{
    if (a == 0.0) return 0.0;
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    int E = ex - 1;                /* a in [2^E, 2^(E+1)) */
    if (E < emin) E = emin;        /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, E - (p - 1));
    double n = rne_nonneg(a / quantum);
    double r = n * quantum;
    /* overflow: anything that rounds above the largest finite value */
    if (r > vmax) return INFINITY;
    return r;
}

/* double -> binary16 bits, round to nearest even, overflow to infinity. */
uint16_t orc_double_to_f16(double v)
{
    if (isnan(v)) return 0x7e00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    double r = round_to_format(a, 11, -14, 65504.0);
    if (isinf(r)) return sign | 0x7c00;
    if (r < ldexp(1.0, -14)) {
        /* subnormal (or zero): fraction = r / 2^-24, an integer < 1024 */
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    }
    int ex;
    frexp(r, &ex);
    int E = ex - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, E - 10) - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | frac;
}

/* double -> bfloat16 bits, round to nearest even, overflow to infinity. */
uint16_t orc_double_to_bf16(double v)
{
    if (isnan(v)) return 0x7fc0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    double vmax = ldexp(255.0, 120);            /* (2 - 2^-7) * 2^127 */
    double r = round_to_format(a, 8, -126, vmax);
    if (isinf(r)) return sign | 0x7f80;
    if (r < ldexp(1.0, -126))
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    int ex;
    frexp(r, &ex);
    int E = ex - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, E - 7) - 128.0);
    return sign | (uint16_t)((E + 127) << 7) | frac;
}

/* OCP FP8 E4M3 ("fn" variant: no infinities, S.1111.111 is NaN), bias 7,
 * subnormals m/8 * 2^-6.  [LUT-B] "Format": codebook entries and MXFP8
 * activation elements are E4M3. */
double orc_e4m3_to_double(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xf;
    int m = b & 0x7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10);        /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* OCP UE8M0 scale: 2^(e-127); 0xFF is NaN.  [LUT-B] "Format": one UE8M0
 * exponent per weight tile; MXFP8 carries one UE8M0 per 32 K. */
double orc_ue8m0_to_double(uint8_t e)
{
    if (e == 0xff) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ------------------------------------------------------------------------ */
/* INT4 group-wise weights.                                                 */
/* ------------------------------------------------------------------------ */

/* Unpack: row n of the weight is stored K-contiguous, two codes per byte.
 * [Metal] step 2: of the two nibbles of a byte, the low one is the weight of
 * the even K row (tid.y*2) and the high one that of the odd K row.  Codes are
 * unsigned 0..15.
 *   codes_out[n][k] = (k even) ? (qweight[n][k/2] & 0xF) : (qweight[n][k/2] >> 4)
 */
void orc_w4_unpack(const uint8_t *qweight, int64_t N, int64_t K, uint8_t *codes_out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = qweight[n * (K / 2) + k / 2];
            codes_out[n * K + k] = (k % 2 == 0) ? (uint8_t)(byte & 0x0f)
                                                : (uint8_t)(byte >> 4);
        }
}

/* Zero point of weight (n, k).
 * Symmetric ([Metal] step 2 subtracts 8 from the unsigned nibble; [ARM] calls
 * this the zero-point-free case): z = 8, i.e. the signed value q-8 in [-8, 7].
 * Asymmetric ([ARM] group-wise quantization: an int8 zero point per group):
 * z = zeros[n][k/G]. */
static int w4_zero(const int8_t *zeros, int64_t n, int64_t k, int64_t K, int G)
{
    if (zeros == NULL) return 8;
    return (int)zeros[n * (K / G) + k / G];
}

/* Dequantize to fp32:  w[n][k] = (q - z) * s[n][k/G].
 * [Metal] step 2 (nibble minus zero point, times the group's scale) and [ARM]
 * group-wise quantization (groups are G consecutive K of one output channel,
 * fp16 scale per group).  The product is formed in double and stored as
 * float: |q - z| <= 143 needs 8 significant bits and an fp16 scale 11, so the
 * product is exact in binary32 and the conversion does not round. */
void orc_w4_dequant(const uint8_t *qweight, const uint16_t *scales, const int8_t *zeros,
                    int64_t N, int64_t K, int G, float *w_out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = qweight[n * (K / 2) + k / 2];
            int q = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
            int z = w4_zero(zeros, n, k, K, G);
            double s = orc_f16_to_double(scales[n * (K / G) + k / G]);
            w_out[n * K + k] = (float)((double)(q - z) * s);
        }
}

/* Activation element m,k as double.  dtype 0 = fp16, 1 = bf16. */
static double act_value(const uint16_t *x, int dtype, int64_t idx)
{
    return dtype == 0 ? orc_f16_to_double(x[idx]) : orc_bf16_to_double(x[idx]);
}

/* y[m][n] = sum_k x[m][k] * w[n][k]  ([Metal] step 3; [ARM]: decode is this
 * product with M = 1, prefill the same product with many rows).
 * Each weight is dequantized as in orc_w4_dequant (exact fp32 value), each
 * product is exact in double, the sum runs in ascending k in double.
 * y64 receives the double sums; y_out (may be NULL) the sums rounded to
 * nearest even in the output type (out_dtype 0 = fp16, 1 = bf16). */
void orc_w4_matmul(const uint16_t *x, int x_dtype, int64_t M, int64_t N, int64_t K, int G,
                   const uint8_t *qweight, const uint16_t *scales, const int8_t *zeros,
                   double *y64, uint16_t *y_out, int out_dtype)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t byte = qweight[n * (K / 2) + k / 2];
                int q = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
                int z = w4_zero(zeros, n, k, K, G);
                double s = orc_f16_to_double(scales[n * (K / G) + k / G]);
                double w = (double)(float)((double)(q - z) * s);
                acc += act_value(x, x_dtype, m * K + k) * w;
            }
            if (y64) y64[m * N + n] = acc;
            if (y_out)
                y_out[m * N + n] = out_dtype == 0 ? orc_double_to_f16(acc)
                                                  : orc_double_to_bf16(acc);
        }
}

/* Same product for a chosen subset of output rows (rows[i] indexes M); used to
 * check full-size prefill products on a sample of rows, which are independent
 * of one another. */
void orc_w4_matmul_rows(const uint16_t *x, int x_dtype, int64_t K, int64_t N, int G,
                        const uint8_t *qweight, const uint16_t *scales, const int8_t *zeros,
                        const int64_t *rows, int64_t n_rows,
                        double *y64, uint16_t *y_out, int out_dtype)
{
    for (int64_t i = 0; i < n_rows; ++i)
        orc_w4_matmul(x + rows[i] * K, x_dtype, 1, N, K, G, qweight, scales, zeros,
                      y64 ? y64 + i * N : NULL, y_out ? y_out + i * N : NULL, out_dtype);
}

/* ------------------------------------------------------------------------ */
/* Uniform b-bit codes, b = 1..8 ([ARM] the 1-8 bit kernel table: one       */
/* unpack routine per bit width; group-wise quantization as for INT4).       */
/* ------------------------------------------------------------------------ */

/* Zero point of a b-bit weight: symmetric 2^(b-1) (the midpoint of the
 * unsigned code range, as z = 8 is for 4 bits), asymmetric the int8 zero
 * point of the group. */
static int wb_zero(const int8_t *zeros, int bits, int64_t n, int64_t k, int64_t K, int G)
{
    if (zeros == NULL) return 1 << (bits - 1);
    return (int)zeros[n * (K / G) + k / G];
}

/* w[n][k] = (q[n][k] - z) * s[n][k/G] with q = codes[n][k] (one code per
 * byte, q < 2^bits); exact in binary32 (|q - z| <= 383 needs 9 bits, an fp16
 * scale 11). */
void orc_wb_dequant(const uint8_t *codes, const uint16_t *scales, const int8_t *zeros, int bits,
                    int64_t N, int64_t K, int G, float *w_out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int q = codes[n * K + k];
            int z = wb_zero(zeros, bits, n, k, K, G);
            double s = orc_f16_to_double(scales[n * (K / G) + k / G]);
            w_out[n * K + k] = (float)((double)(q - z) * s);
        }
}

/* y[m][n] = sum_k x[m][k] * w[n][k], x fp16, ascending k in double (every
 * product exact), y_out fp16 RNE (may be NULL). */
void orc_wb_matmul(const uint16_t *x, int64_t M, int64_t N, int64_t K, int G, int bits,
                   const uint8_t *codes, const uint16_t *scales, const int8_t *zeros,
                   double *y64, uint16_t *y_out)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int q = codes[n * K + k];
                int z = wb_zero(zeros, bits, n, k, K, G);
                double s = orc_f16_to_double(scales[n * (K / G) + k / G]);
                acc += orc_f16_to_double(x[m * K + k]) * ((double)(q - z) * s);
            }
            if (y64) y64[m * N + n] = acc;
            if (y_out) y_out[m * N + n] = orc_double_to_f16(acc);
        }
}

/* ------------------------------------------------------------------------ */
/* 3-bit LUT-codebook MoE with MXFP8 activations.                           */
/* ------------------------------------------------------------------------ */

/* Weight of expert e at (n, k):
 *   w_e[n][k] = E4M3(cb[e][n/8][k/64][idx_e[n][k]]) * 2^(ex[e][n/8][k/64] - 127)
 * [LUT-B] "Format": each weight is a 3-bit index into an 8-entry E4M3
 * codebook; one codebook and one UE8M0 exponent are shared by a tile of
 * 8 output channels x 64 K.  Readings: codebook position = index value 0..7;
 * the exponent multiplies the decoded entry. */
static double lut3_weight(const uint8_t *idx, const uint8_t *cb, const uint8_t *ex,
                          int64_t e, int64_t n, int64_t k, int64_t N, int64_t K)
{
    int64_t tiles_k = K / 64;
    int64_t tile = (e * (N / 8) + n / 8) * tiles_k + k / 64;
    uint8_t i = idx[(e * N + n) * K + k];
    return orc_e4m3_to_double(cb[tile * 8 + i]) * orc_ue8m0_to_double(ex[tile]);
}

/* Dequantize all experts to double: w_out[e][n][k]. */
void orc_lut3_dequant(const uint8_t *idx, const uint8_t *cb, const uint8_t *ex,
                      int64_t E, int64_t N, int64_t K, double *w_out)
{
    for (int64_t e = 0; e < E; ++e)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < K; ++k)
                w_out[(e * N + n) * K + k] = lut3_weight(idx, cb, ex, e, n, k, N, K);
}

/* MXFP8 activation element: E4M3(aq[r][k]) * 2^(as[r][k/32] - 127)
 * ([LUT-B] "Motivation": E4M3 values with one UE8M0 scale per 1x32 K). */
static double mx_act(const uint8_t *aq, const uint8_t *as, int64_t r, int64_t k, int64_t K)
{
    return orc_e4m3_to_double(aq[r * K + k]) * orc_ue8m0_to_double(as[r * (K / 32) + k / 32]);
}

/* Routing bucketing ([LUT-B] "A gather": rows are visited through
 * sorted_token_ids built by moe_align_block_size; a slot is valid when its id
 * is below num_valid_tokens).  Readings taken where the page is silent:
 *   - slot id sid = t * top_k + j for token t and its j-th routed expert;
 *   - experts are visited in ascending global id; within an expert, sids in
 *     ascending order; each expert's list is padded with the sentinel
 *     T*top_k up to a multiple of block_m; experts with no slot get no block;
 *   - block_expert[b] = expert_map[e] (local id, -1 if not local; identity
 *     when expert_map is NULL) for every block of expert e.
 * Returns the padded length; writes at most `cap` sorted ids and cap/block_m
 * block entries (returns -1 if cap is too small). */
int64_t orc_moe_align(const int32_t *topk_ids, int64_t T, int64_t top_k, int64_t E,
                      int64_t block_m, const int32_t *expert_map,
                      int32_t *sorted_ids, int32_t *block_expert, int64_t cap)
{
    int64_t num_valid = T * top_k;
    int64_t pos = 0;
    for (int64_t e = 0; e < E; ++e) {
        int64_t count = 0;
        for (int64_t sid = 0; sid < num_valid; ++sid)
            if (topk_ids[sid] == e) {
                if (pos + count >= cap) return -1;
                sorted_ids[pos + count] = (int32_t)sid;
                ++count;
            }
        if (count == 0) continue;
        int64_t padded = ((count + block_m - 1) / block_m) * block_m;
        if (pos + padded > cap) return -1;
        for (int64_t i = count; i < padded; ++i)
            sorted_ids[pos + i] = (int32_t)num_valid;
        for (int64_t b = pos / block_m; b < (pos + padded) / block_m; ++b)
            block_expert[b] = expert_map ? expert_map[e] : (int32_t)e;
        pos += padded;
    }
    return pos;
}

/* Grouped expert product, the emulation-path numerics of [LUT-B] "Emulation
 * path" carried out in double:
 *   for every slot sid < T*top_k with global expert g = topk_ids[sid] and
 *   local expert e = expert_map[g] (identity when NULL):
 *     e < 0  : out[sid][:] = 0            ([LUT-B] "Expert parallelism")
 *     else   : y64[sid][n] = sum_k a[row(sid)][k] * w_e[n][k], ascending k,
 *              out[sid][n] = RNE_bf16(y64)
 *   row(sid) = sid / a_row_div  (a_row_div = top_k when every routed copy of a
 *   token reads the token's hidden row, 1 when each slot has its own row).
 * Every decoded value and product is exact in double. */
void orc_moe_gemm(const uint8_t *idx, const uint8_t *cb, const uint8_t *ex,
                  int64_t E_local, int64_t N, int64_t K,
                  const uint8_t *aq, const uint8_t *as, int64_t a_row_div,
                  const int32_t *topk_ids, int64_t T, int64_t top_k,
                  const int32_t *expert_map,
                  double *y64, uint16_t *out_bf16)
{
    int64_t num_valid = T * top_k;
    for (int64_t sid = 0; sid < num_valid; ++sid) {
        int32_t g = topk_ids[sid];
        int32_t e = expert_map ? expert_map[g] : g;
        int64_t r = sid / a_row_div;
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            if (e >= 0 && e < E_local)
                for (int64_t k = 0; k < K; ++k)
                    acc += mx_act(aq, as, r, k, K) * lut3_weight(idx, cb, ex, e, n, k, N, K);
            if (y64) y64[sid * N + n] = acc;
            if (out_bf16) out_bf16[sid * N + n] = orc_double_to_bf16(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* W4A8: the same INT4 weights against dynamically quantized INT8            */
/* activations ([ARM] measurements section: 4-bit weights with dynamic INT8  */
/* activations, group size 32; the inner loop keeps unpacked weights as int8 */
/* and feeds int8 matrix-multiply instructions with int32 accumulation).    */
/* ------------------------------------------------------------------------ */

/* Per-token dynamic INT8 quantization of fp16 activations.
 * The page names the scheme only.  Readings: one scale per token row,
 * symmetric, codes in [-127, 127], the row's largest magnitude mapping to
 * 127.  The decisions that produce integers are taken in binary32, the
 * precision the GPU takes them in, with every operation correctly rounded:
 *   amax = max_k |x[m][k]|                 (exact)
 *   inv  = fl32(127 / amax)
 *   q    = rint(fl32(x[m][k] * inv))       (ties to even; |q| <= 127 always,
 *                                           clamped for clarity)
 *   s    = fl32(amax / 127)                (the dequantization scale)
 * A row of zeros gets s = 0 and all codes 0.  x must be finite. */
void orc_quant_act_i8(const uint16_t *x, int64_t M, int64_t K, int8_t *xq, float *sx)
{
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf((float)orc_f16_to_double(x[m * K + k]));
            if (v > amax) amax = v;
        }
        float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        sx[m] = amax / 127.0f;
        for (int64_t k = 0; k < K; ++k) {
            float t = (float)orc_f16_to_double(x[m * K + k]) * inv;
            float r = rintf(t);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            xq[m * K + k] = (int8_t)r;
        }
    }
}

/* y[m][n] = sum_k (s[m] * xq[m][k]) * w[n][k]:  the INT4 weights of
 * orc_w4_dequant against the dequantized INT8 activations of
 * orc_quant_act_i8.  Every term is exact in double (s: 24 significant bits,
 * xq: 8, w: 19); the sum runs in ascending k in double and is rounded to
 * nearest even into fp16 (y_out, may be NULL). */
void orc_w4a8_matmul(const uint16_t *x, int64_t M, int64_t N, int64_t K, int G,
                     const uint8_t *qweight, const uint16_t *scales, const int8_t *zeros,
                     double *y64, uint16_t *y_out)
{
    int8_t *xq = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    float *sx = (float *)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    if (!xq || !sx) { free(xq); free(sx); return; }
    orc_quant_act_i8(x, M, K, xq, sx);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t byte = qweight[n * (K / 2) + k / 2];
                int q = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
                int z = w4_zero(zeros, n, k, K, G);
                double s = orc_f16_to_double(scales[n * (K / G) + k / G]);
                double w = (double)(q - z) * s;
                double a = (double)sx[m] * (double)xq[m * K + k];
                acc += a * w;
            }
            if (y64) y64[m * N + n] = acc;
            if (y_out) y_out[m * N + n] = orc_double_to_f16(acc);
        }
    free(xq);
    free(sx);
}

/* ------------------------------------------------------------------------ */
/* The MoE layer around the two grouped GEMMs: SiLU(gate) * up, MXFP8       */
/* re-quantization of the result, router-weighted combine of the experts'   */
/* outputs.  The page (section "Emulation path") runs the experts on MXFP8  */
/* activations quantized before each GEMM; it does not spell these steps    */
/* out, so each reading is stated where it is used.                        */
/* ------------------------------------------------------------------------ */

/* double -> OCP E4M3 byte (1 sign, 4 exponent bits with bias 7, 3 fraction
 * bits; largest finite 448), round to nearest even, saturating: magnitudes
 * that round above 448 give 448 (the MX conversion clamps to the largest
 * normal; E4M3 has no infinity).  NaN -> 0x7F. */
uint8_t orc_double_to_e4m3(double v)
{
    if (isnan(v)) return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double r = round_to_format(fabs(v), 4, -6, 448.0);
    if (isinf(r)) r = 448.0;
    if (r < ldexp(1.0, -6))                          /* subnormal or zero: r / 2^-9 */
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    int ex;
    frexp(r, &ex);
    int E = ex - 1;                                  /* r in [2^E, 2^(E+1)), -6 <= E <= 8 */
    int frac = (int)(r / ldexp(1.0, E - 3)) - 8;     /* 0..7 */
    return sign | (uint8_t)(((E + 7) << 3) | frac);
}

/* MXFP8 quantization (OCP MX: one shared power-of-two scale per 32
 * consecutive elements of a row, elements in E4M3).  Reading: the shared
 * exponent is floor(log2(amax)) - 8, 8 being the exponent of E4M3's largest
 * value, clamped to the UE8M0 range [-127, 127]; each element becomes the
 * saturating round-to-nearest-even E4M3 of x / 2^e; an all-zero block gets
 * exponent 0 (byte 127).  x: bf16 bits [R][K], K % 32 == 0; q: u8 [R][K];
 * s: u8 [R][K/32] (UE8M0 = e + 127). */
void orc_mxfp8_quant(const uint16_t *x, int64_t R, int64_t K, uint8_t *q, uint8_t *s)
{
    for (int64_t r = 0; r < R; ++r)
        for (int64_t b = 0; b < K / 32; ++b) {
            double amax = 0.0;
            for (int64_t k = 32 * b; k < 32 * b + 32; ++k) {
                double v = fabs(orc_bf16_to_double(x[r * K + k]));
                if (v > amax) amax = v;
            }
            int e = 0;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);                    /* amax = m * 2^ex, m in [0.5, 1) */
                e = (ex - 1) - 8;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            s[r * (K / 32) + b] = (uint8_t)(e + 127);
            for (int64_t k = 32 * b; k < 32 * b + 32; ++k)
                q[r * K + k] = orc_double_to_e4m3(ldexp(orc_bf16_to_double(x[r * K + k]), -e));
        }
}

/* 2^t in binary32 by a stated algorithm (the layer's SiLU uses it on both
 * sides, so the E4M3 codes that follow compare bit for bit): n = rint(t)
 * (ties to even), f = t - n (exact, |f| <= 1/2), 2^f = e^(f ln 2) by its
 * Taylor polynomial through degree 7 evaluated in Horner form with
 * correctly rounded fused multiply-adds, then scaled by 2^n.  t is first
 * clamped to [-100, 100], so every result is a normal binary32 number.  The
 * coefficients are (ln 2)^k / k! rounded to binary32. */
static float exp2_f32(float t)
{
    static const double LN2 = 0.693147180559945309417232121458;
    if (t > 100.0f) t = 100.0f;
    if (t < -100.0f) t = -100.0f;
    float n = rintf(t);
    float f = t - n;
    float c[8];
    double term = 1.0;
    for (int k = 0; k < 8; ++k) {                    /* (ln 2)^k / k! */
        c[k] = (float)term;
        term = term * LN2 / (double)(k + 1);
    }
    float p = c[7];
    for (int k = 6; k >= 0; --k) p = fmaf(p, f, c[k]);
    return ldexpf(p, (int)n);
}

/* SiLU(g) = g / (1 + e^-g), in binary32: e^-g = 2^(fl32(-g * fl32(log2 e)))
 * by exp2_f32, then fl32(1 + e), fl32(1 / that), fl32(g * that). */
float orc_silu_f32(float g)
{
    const float LOG2E = 1.44269504088896340736f;
    float t = -g * LOG2E;
    float e = exp2_f32(t);
    float sig = 1.0f / (1.0f + e);
    return g * sig;
}

/* act[r][j] = RNE_bf16( fl32( SiLU(gate) * up ) ), gate = gu[r][j],
 * up = gu[r][I + j] (the gate/up GEMM stacks the two projections along N:
 * columns 0..I-1 gate, I..2I-1 up).  gu, act: bf16 bits. */
void orc_silu_mul_bf16(const uint16_t *gu, int64_t R, int64_t I, uint16_t *act)
{
    for (int64_t r = 0; r < R; ++r)
        for (int64_t j = 0; j < I; ++j) {
            float g = (float)orc_bf16_to_double(gu[r * 2 * I + j]);
            float u = (float)orc_bf16_to_double(gu[r * 2 * I + I + j]);
            float a = orc_silu_f32(g) * u;
            act[r * I + j] = orc_double_to_bf16((double)a);
        }
}

/* Router-weighted combine of the routed experts' outputs:
 *   y64[t][h] = sum_{j < top_k} w[t][j] * out[t * top_k + j][h]
 * in double, ascending j (every product is exact: 24 + 8 significant bits),
 * y_bf16 = RNE_bf16(y64).  A slot of an expert that is not local has a zero
 * row in `out` and adds nothing.  out: bf16 bits [T*top_k][H]; w: f32. */
void orc_moe_combine(const uint16_t *out, const float *w, int64_t T, int64_t top_k, int64_t H,
                     double *y64, uint16_t *y_bf16)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t j = 0; j < top_k; ++j)
                acc += (double)w[t * top_k + j] * orc_bf16_to_double(out[(t * top_k + j) * H + h]);
            if (y64) y64[t * H + h] = acc;
            if (y_bf16) y_bf16[t * H + h] = orc_double_to_bf16(acc);
        }
}

void orc_silu_f32_array(const float *g, int64_t n, float *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_silu_f32(g[i]); }

void orc_exp2_f32_array(const float *t, int64_t n, float *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = exp2_f32(t[i]); }

void orc_double_array_to_e4m3(const double *v, int64_t n, uint8_t *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_e4m3(v[i]); }

/* ------------------------------------------------------------------------ */
/* Array forms of the format conversions (one call per array, for tests).   */
/* ------------------------------------------------------------------------ */

void orc_f16_array_to_double(const uint16_t *h, int64_t n, double *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_double(h[i]); }

void orc_bf16_array_to_double(const uint16_t *b, int64_t n, double *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_double(b[i]); }

void orc_double_array_to_f16(const double *v, int64_t n, uint16_t *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_f16(v[i]); }

void orc_double_array_to_bf16(const double *v, int64_t n, uint16_t *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_bf16(v[i]); }

void orc_e4m3_array_to_double(const uint8_t *b, int64_t n, double *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_to_double(b[i]); }

void orc_ue8m0_array_to_double(const uint8_t *b, int64_t n, double *out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_ue8m0_to_double(b[i]); }

/* Version tag so a caller can check it loaded this file's build. */
int orc_version(void) { return 1; }
