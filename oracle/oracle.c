/*
 * CPU oracle for the weight-only 4-bit dequantize-and-multiply path,
 * y = x . dequant(W)^T, in its three weight encodings.
 *
 * TEST INFRASTRUCTURE. This file is the independent, deliberately plain
 * reference that the HIP library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may build, load or
 * call it; the product path never does. It shares no code, header, table
 * or helper with the HIP library: every conversion below is written here
 * from its format definition.
 *
 * Conventions:
 *   - floating point stays in the precision the pages state; products and
 *     sums of the contraction are carried in double (fp64) and summed in
 *     ascending k, so the accumulator is the exact dot product up to the
 *     fp64 rounding of a K-term sum;
 *   - build with -ffp-contract=off so every f32 expression rounds exactly
 *     as written;
 *   - OpenMP parallelises over independent output elements only.
 *
 * Sources (the three pages this oracle follows):
 *   [P1] onnxruntime-ep-mlx 0.27.4, src/ops/quant_fastkernel.rs - INT4
 *        group-32 affine MatMulNBits: module doc ("Algorithm"), the kernel
 *        SOURCE (W load), and the tests' make_case host ground truth.
 *   [P2] onnxruntime-ep-mlx 0.31.1, src/ops/lut4.rs - frozen 16-entry
 *        lookup decode: the decode kernel in decoded_gemm, the CPU branch
 *        of execute, rounded_weight, and the recognize() rounding rule.
 *   [P3] mlx-native 0.9.0, src/ops/quantized_matmul_id_ggml.rs - the
 *        expert-routed contraction stated in the module doc, over GGML
 *        Q4_0 blocks.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* 16-bit float formats, written from their definitions.               */
/* ------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE-754 binary32 word. */
float w4o_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even, on the 16 dropped
 * bits. A NaN stays a (quiet) NaN with its sign. */
uint16_t w4o_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (upper & 1u)))
        upper += 1u; /* a carry into the exponent rounds up to the next binade or to inf */
    return (uint16_t)upper;
}

/* IEEE-754 binary16 -> value: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is subnormal (fraction * 2^-24), exponent 31 is
 * inf/NaN. The double result is exact and fits binary32 exactly. */
float w4o_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

/* value -> binary16, round to nearest, ties to even. The input is an exact
 * binary32 value; it is written as n * 2^(e-10) with the quantum of its
 * binade (clamped to the subnormal quantum 2^-24) and n rounded to an
 * integer, ties to even. */
uint16_t w4o_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)f);
    if (isinf(f))
        return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e); /* a = fr * 2^e, fr in [0.5, 1) -> a in [2^(e-1), 2^e) */
    e -= 1;             /* now a in [2^e, 2^(e+1)) */
    if (e < -14)
        e = -14;        /* subnormal range shares the quantum 2^-24 */
    double quantum = ldexp(1.0, e - 10);
    double n = a / quantum;      /* exact: power-of-two division */
    double fl = floor(n);
    double diff = n - fl;
    if (diff > 0.5 || (diff == 0.5 && fmod(fl, 2.0) != 0.0))
        fl += 1.0;
    if (fl >= 2048.0) { /* rounded up into the next binade */
        fl = 1024.0;
        e += 1;
    }
    if (e > 15)
        return (uint16_t)(sign | 0x7C00u); /* overflow -> inf */
    if (fl < 1024.0)                          /* subnormal (only when e == -14) */
        return (uint16_t)(sign | (uint16_t)fl);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(fl - 1024.0));
}

/* Bulk forms, so the Python side can use this file's conversions alone. */
void w4o_bf16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_bf16_to_f32(in[i]);
}
void w4o_f32_to_bf16_n(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_f32_to_bf16(in[i]);
}
void w4o_f16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_f16_to_f32(in[i]);
}
void w4o_f32_to_f16_n(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = w4o_f32_to_f16(in[i]);
}

/* ------------------------------------------------------------------ */
/* Affine INT4 (P1).                                                    */
/* ------------------------------------------------------------------ */

/* P1, kernel SOURCE (W load) and make_case: W is [N, K/8] uint32; the
 * weight at (n, k) is nibble j = k % 8 of word k / 8, taken least
 * significant nibble first (bits 4j..4j+3). */
static inline uint32_t affine_nibble(const uint32_t* w, int64_t K, int64_t n, int64_t k)
{
    uint32_t word = w[n * (K / 8) + k / 8];
    return (word >> (4 * (k % 8))) & 0xFu;
}

void w4o_unpack_affine(const uint32_t* w, int64_t N, int64_t K, uint8_t* q)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = (uint8_t)affine_nibble(w, K, n, k);
}

/* P1 module doc and make_case: w = q * scale + bias per group of `group`
 * consecutive k, scales/biases [N, K/group] bf16 (bias already -zp*scale).
 * q*scale is exact in f32 (4-bit times 8-bit significand); the add rounds
 * once, as the page's host ground truth does. */
static inline float affine_weight(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                                  int64_t K, int64_t group, int64_t n, int64_t k)
{
    int64_t groups = K / group;
    float s = w4o_bf16_to_f32(scales[n * groups + k / group]);
    float b = w4o_bf16_to_f32(biases[n * groups + k / group]);
    float q = (float)affine_nibble(w, K, n, k);
    float qs = q * s;
    return qs + b;
}

void w4o_dequant_affine(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                        int64_t N, int64_t K, int64_t group, float* W)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = affine_weight(w, scales, biases, K, group, n, k);
}

/* y[m][n] = sum_k x[m][k] * W[n][k]; x bf16 [M, K], y bf16 [M, N] (P1 module
 * doc: the output is bf16, one rounding of the f32 accumulator, here RNE of
 * the f32-rounded fp64 sum). acc (optional) receives the fp64 sums. */
void w4o_affine(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                const uint16_t* x, int64_t M, int64_t K, int64_t N, int64_t group,
                double* acc, uint16_t* y)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = (double)w4o_bf16_to_f32(x[m * K + k]);
                double wv = (double)affine_weight(w, scales, biases, K, group, n, k);
                s += xv * wv;
            }
            if (acc) acc[m * N + n] = s;
            if (y) y[m * N + n] = w4o_f32_to_bf16((float)s);
        }
    }
}

/* The same sums for a list of (m, n) points only, for checks at full size. */
void w4o_affine_points(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, int64_t K, int64_t group,
                       const int64_t* ms, const int64_t* ns, int64_t count,
                       double* acc, uint16_t* y)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += (double)w4o_bf16_to_f32(x[m * K + k]) *
                 (double)affine_weight(w, scales, biases, K, group, n, k);
        if (acc) acc[i] = s;
        if (y) y[i] = w4o_f32_to_bf16((float)s);
    }
}

/* ------------------------------------------------------------------ */
/* Lookup-codebook 4-bit (P2).                                          */
/* ------------------------------------------------------------------ */

/* P2 decode kernel / CPU branch: flat index i over the decoded [rows, cols]
 * matrix; code = high nibble of packed[i/2] when i is even, low nibble when
 * i is odd. */
static inline uint32_t lut_code(const uint8_t* packed, int64_t i)
{
    uint32_t byte = packed[i / 2];
    return (i % 2 == 0) ? (byte >> 4) : (byte & 15u);
}

void w4o_unpack_lut(const uint8_t* packed, int64_t count, uint8_t* codes)
{
    for (int64_t i = 0; i < count; ++i) codes[i] = (uint8_t)lut_code(packed, i);
}

/* P2: weight[i] = book[code(i)] * scales[i / block] in f32; when the graph
 * casts the decoded weight to half (rounding == HALF), it is rounded to
 * binary16 before the matmul (rounded_weight). Blocks run over the flat
 * index and may straddle rows. */
void w4o_lut_decode(const uint8_t* packed, const float* scales, const float* book,
                    int64_t rows, int64_t cols, int64_t block, int round_half, float* W)
{
    int64_t count = rows * cols;
    for (int64_t i = 0; i < count; ++i) {
        float v = book[lut_code(packed, i)] * scales[i / block];
        if (round_half) v = w4o_f16_to_f32(w4o_f32_to_f16(v));
        W[i] = v;
    }
}

/* P2 decoded_weight_gemm / CPU branch: y = x @ W^T when transpose (W is
 * [rows = N, cols = K]), else y = x @ W (W is [rows = K, cols = N]).
 * x f32 [M, K]; acc fp64 [M, N]. */
void w4o_lut_matmul(const float* x, const float* W, int64_t M, int64_t K, int64_t N,
                    int transpose, double* acc)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                float wv = transpose ? W[n * K + k] : W[k * N + n];
                s += (double)x[m * K + k] * (double)wv;
            }
            acc[m * N + n] = s;
        }
}

/* Full-size point checks (transpose layout, fp16 scales and x as stored). */
void w4o_lut_points(const uint16_t* x_f16, const uint8_t* packed, const uint16_t* scales_f16,
                    const float* book, int64_t K, int64_t block, int round_half,
                    const int64_t* ms, const int64_t* ns, int64_t count, double* acc)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t flat = n * K + k;
            float v = book[lut_code(packed, flat)] * w4o_f16_to_f32(scales_f16[flat / block]);
            if (round_half) v = w4o_f16_to_f32(w4o_f32_to_f16(v));
            s += (double)w4o_f16_to_f32(x_f16[m * K + k]) * (double)v;
        }
        acc[i] = s;
    }
}

/* ------------------------------------------------------------------ */
/* Expert-routed GGML Q4_0 (P3).                                        */
/* ------------------------------------------------------------------ */

/* GGML Q4_0 block (the pages name the format but do not spell out its
 * bytes; this is the published layout): 18 bytes = little-endian binary16
 * scale d, then 16 bytes qs. Element i < 16 of the block is the low nibble
 * of qs[i], element i + 16 its high nibble; value = (q - 8) * d. */
enum { Q4_0_QK = 32, Q4_0_BYTES = 18 };

static inline const uint8_t* q4_0_block(const uint8_t* w, uint64_t expert_stride, int64_t K,
                                        int64_t e, int64_t n, int64_t j)
{
    int64_t row_bytes = (K / Q4_0_QK) * Q4_0_BYTES;
    return w + (uint64_t)e * expert_stride + (uint64_t)(n * row_bytes + j * Q4_0_BYTES);
}

static inline uint32_t q4_0_code(const uint8_t* blk, int64_t i)
{
    return (i < 16) ? (blk[2 + i] & 0xFu) : (blk[2 + (i - 16)] >> 4);
}

static inline float q4_0_scale(const uint8_t* blk)
{
    return w4o_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* rows consecutive weight rows starting at w (one expert slab or any row
 * range), K values each: q[rows, K] codes and d[rows, K/32] scales. */
void w4o_unpack_q4_0(const uint8_t* w, int64_t rows, int64_t K, uint8_t* q, float* d)
{
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t j = 0; j < K / Q4_0_QK; ++j) {
            const uint8_t* blk = q4_0_block(w, 0, K, 0, n, j);
            if (d) d[n * (K / Q4_0_QK) + j] = q4_0_scale(blk);
            for (int64_t i = 0; i < Q4_0_QK; ++i) q[n * K + j * Q4_0_QK + i] = (uint8_t)q4_0_code(blk, i);
        }
}

static inline float q4_0_weight(const uint8_t* w, uint64_t expert_stride, int64_t K,
                                int64_t e, int64_t n, int64_t k)
{
    const uint8_t* blk = q4_0_block(w, expert_stride, K, e, n, k / Q4_0_QK);
    float q = (float)((int)q4_0_code(blk, k % Q4_0_QK) - 8);
    return q * q4_0_scale(blk); /* exact: 4-bit integer times 11-bit significand */
}

/* P3 module doc: for each (token, slot) row r = token * top_k + slot,
 * expert = ids[r] and out[r][n] = sum_k dequant(W[expert][n][k]) * x[token][k].
 * x f32 [n_tokens, K]; out f32 [n_tokens * top_k, N]. A row whose id is not
 * below n_experts has no expert to read: it is written as zeros (the pages
 * leave this case open). acc (optional) receives the fp64 sums. */
void w4o_moe_q4_0(const float* x, const uint8_t* w, const uint32_t* ids,
                  int64_t n_tokens, int64_t top_k, int64_t N, int64_t K, int64_t n_experts,
                  uint64_t expert_stride, double* acc, float* out)
{
    int64_t rows = n_tokens * top_k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t e = ids[r];
        int64_t t = r / top_k;
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            if (e < n_experts)
                for (int64_t k = 0; k < K; ++k)
                    s += (double)x[t * K + k] * (double)q4_0_weight(w, expert_stride, K, e, n, k);
            if (acc) acc[r * N + n] = s;
            if (out) out[r * N + n] = (float)s;
        }
    }
}

/* Point checks for (row r, column n) pairs. */
/* P3 quantized_matmul_id_swiglu_q4_0 doc: for each routed row r, expert
 * e = ids[r] and out[r][n] = sum_k dequant(W[e][n][k]) * (silu(gate[r][k]) *
 * up[r][k]), where gate and up are per routed row (f32 [rows, K]) and
 * silu(g) = g * sigmoid(g) = g / (1 + e^-g). The activation product is
 * formed in double from the f32 inputs. Out-of-range ids give zero rows, as
 * in w4o_moe_q4_0. */
static double silu(double g)
{
    return g / (1.0 + exp(-g)); /* g -> -inf: exp overflows to inf and the quotient is -0 */
}

void w4o_moe_swiglu_q4_0(const float* gate, const float* up, const uint8_t* w, const uint32_t* ids,
                         int64_t rows, int64_t N, int64_t K, int64_t n_experts, uint64_t expert_stride,
                         double* acc, float* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t e = ids[r];
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            if (e < n_experts)
                for (int64_t k = 0; k < K; ++k) {
                    double a = silu((double)gate[r * K + k]) * (double)up[r * K + k];
                    s += a * (double)q4_0_weight(w, expert_stride, K, e, n, k);
                }
            if (acc) acc[r * N + n] = s;
            if (out) out[r * N + n] = (float)s;
        }
    }
}

void w4o_moe_q4_0_points(const float* x, const uint8_t* w, const uint32_t* ids, int64_t top_k,
                         int64_t K, int64_t n_experts, uint64_t expert_stride,
                         const int64_t* rs, const int64_t* ns, int64_t count, double* acc)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < count; ++i) {
        int64_t r = rs[i], n = ns[i];
        int64_t e = ids[r], t = r / top_k;
        double s = 0.0;
        if (e < n_experts)
            for (int64_t k = 0; k < K; ++k)
                s += (double)x[t * K + k] * (double)q4_0_weight(w, expert_stride, K, e, n, k);
        acc[i] = s;
    }
}
