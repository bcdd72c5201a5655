/*
 * qref.c -- CPU oracle for the weight-only quantized GEMM (fpA_intB) and its
 * top-k MoE variant.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition the GPU path is checked against.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the HIP library; neither includes the other.
 *
 * Every floating-point reduction accumulates in double, except the two
 * qref_gemm_*_f32acc functions, which carry the same sums in fp32 (the
 * timed CPU baseline).  Nothing is blocked, fused or reordered beyond the
 * definitions cited at each function.
 *
 * Sources (the three web pages this work is built from):
 *   [acext]   "acext User Guide (v1.7)": 1.2.1 fpAintB GEMM (argument set of
 *             gemm: A, B, scales, zero points, biases, C, m, n, k, group size),
 *             1.2.3 MoE GEMM (runMoe arguments), 1.3.1 Int8 Weight-only
 *             (one scale per output channel), 1.3.3 Int4 Groupwise (groups of
 *             64 or 128 along K, each with its own scale; zeros for
 *             asymmetric grids).
 *   [allspark] "[Misc][Kernel]: Add GPTQAllSpark Quantization" (vLLM PR 12931),
 *             PR description: A16W8 with group size -1 (per-channel).
 *   [cpuint4] vllm-omni cpu_int4.py: module docstring (checkpoint format
 *             weight_packed uint8 [N, K/2], byte j = w[2j] | w[2j+1] << 4,
 *             bf16 scale/zero [N, K/group], w = (q - 8) * scale + zero),
 *             pack_nibbles / unpack_nibbles, quantize_groupwise (min/max
 *             grid per group), CPUInt4EmbeddingMethod.embedding
 *             (dequantize in fp32, then cast), CPUInt4LinearMethod.apply
 *             (bias added after the GEMM).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - scale, zero and A share one dtype (bf16 or fp16); bias has its own.
 *   - int8 codes are signed two's complement, stored [N, K] row-major.
 *   - group_size -1 (or K) means one scale per output channel.
 *   - the dequantized weight is an fp32 value; (q-8)*s is exact in fp32, so
 *     only the add of the zero rounds (round-to-nearest-even).
 *   - MoE: top-k over the raw fp32 logits (softmax is monotone), ties to the
 *     lower expert index; weights are the softmax over the k selected logits;
 *     fc1 rows [0, I) are the gate and [I, 2I) the up projection; the
 *     activation is silu(gate) * up with silu(x) = x / (1 + exp(-x)).
 *
 * Dtype codes (same numbering as the library's, written out independently):
 *   0 = none, 1 = bf16, 2 = fp16.  16-bit floats are passed as raw bit
 *   patterns (uint16_t).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QREF_NONE 0
#define QREF_BF16 1
#define QREF_FP16 2

/* Threads: the OpenMP loops below run on omp_get_max_threads() threads
 * unless qref_set_threads() picked a count; qref_team_size() reports the
 * size of the team a parallel region actually gets (what a timing used). */
int qref_threads(void) { return omp_get_max_threads(); }
void qref_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int qref_team_size(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        t = omp_get_num_threads();
    }
    return t;
}

/* ---------------------------------------------------------------------- */
/* 16-bit float <-> fp32, from the IEEE-754 / bfloat16 bit definitions.     */
/* ---------------------------------------------------------------------- */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the top half of an fp32 pattern: widening is exact. */
float qref_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float qref_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t f = (uint32_t)h & 0x3FFu;
    double mag;
    if (e == 0x1F) {
        if (f) return bits_to_f32(0x7FC00000u | (sign << 31));
        return bits_to_f32(0x7F800000u | (sign << 31));
    }
    if (e == 0) mag = ldexp((double)f, -24);                 /* subnormal */
    else        mag = ldexp((double)(f | 0x400u), (int)e - 25);
    return (float)(sign ? -mag : mag);                       /* exact */
}

/* fp32 -> bfloat16, round to nearest, ties to even (NaN stays NaN). */
uint16_t qref_f32_to_bf16(float x)
{
    uint32_t u = f32_to_bits(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16, rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

/* fp32 -> binary16, round to nearest, ties to even, overflow to inf.
 * Written as: pick the binade's quantum, round |x| to a multiple of it. */
uint16_t qref_f32_to_f16(float x)
{
    uint32_t u = f32_to_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if ((u & 0x7F800000u) == 0x7F800000u)
        return (uint16_t)(sign | 0x7C00u | ((u & 0x007FFFFFu) ? 0x200u : 0u));
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                      /* a = m * 2^e, m in [0.5, 1) */
    int exp_unbiased = e - 1;          /* a in [2^eu, 2^(eu+1)) */
    if (exp_unbiased < -14) exp_unbiased = -14;   /* subnormal quantum */
    double quantum = ldexp(1.0, exp_unbiased - 10);
    double q = a / quantum;            /* exact: power-of-two divide */
    double fl = floor(q), diff = q - fl;
    double r = fl;
    if (diff > 0.5 || (diff == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
    double v = r * quantum;
    if (v >= 65536.0 - 16.0) return (uint16_t)(sign | 0x7C00u);  /* >= 65520: inf */
    /* encode v (a multiple of quantum, representable) */
    if (v < ldexp(1.0, -14)) {
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
    }
    int e2;
    double m2 = frexp(v, &e2);         /* v = m2 * 2^e2 */
    uint32_t biased = (uint32_t)(e2 - 1 + 15);
    uint32_t frac = (uint32_t)((m2 * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (biased << 10) | frac);
}

static double act_to_double(uint16_t h, int dtype)
{
    return dtype == QREF_FP16 ? (double)qref_f16_to_f32(h) : (double)qref_bf16_to_f32(h);
}

static float act_to_f32(uint16_t h, int dtype)
{
    return dtype == QREF_FP16 ? qref_f16_to_f32(h) : qref_bf16_to_f32(h);
}

/* ---------------------------------------------------------------------- */
/* Nibble packing  [cpuint4] pack_nibbles / unpack_nibbles, format in the    */
/* module docstring: byte j of a row holds code 2j (low) and 2j+1 (high).    */
/* ---------------------------------------------------------------------- */

void qref_pack4(const int32_t *codes, uint8_t *packed, int64_t n, int64_t k)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k / 2; ++j) {
            uint32_t lo = (uint32_t)codes[r * k + 2 * j] & 0xFu;
            uint32_t hi = (uint32_t)codes[r * k + 2 * j + 1] & 0xFu;
            packed[r * (k / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

void qref_unpack4(const uint8_t *packed, int32_t *codes, int64_t n, int64_t k)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            uint8_t byte = packed[r * (k / 2) + c / 2];
            codes[r * k + c] = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        }
}

/* ---------------------------------------------------------------------- */
/* Groupwise min/max 4-bit quantizer  [cpuint4] quantize_groupwise.  For    */
/* each K-group of a row, with lo / hi its smallest / largest value:        */
/*   scale = max(hi - lo, 1e-9) / 15,  zero = lo + 8 * scale,               */
/*   q = round((w - lo) / scale), ties to even, clamped to [0, 15],         */
/* so that (q - 8) * scale + zero gives lo at q = 0 and hi at q = 15 (the   */
/* docstring's grid).  Every step in fp32, as the page's float tensors;     */
/* codes packed as pack_nibbles.  rintf rounds to nearest even under the    */
/* default floating-point environment, like torch's round.                  */
/* ---------------------------------------------------------------------- */
void qref_quantize4(const float *w, int64_t n, int64_t k, int64_t group, uint8_t *packed,
                    float *scale, float *zero)
{
    int64_t ngroups = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < ngroups; ++g) {
            const float *x = w + r * k + g * group;
            float lo = x[0], hi = x[0];
            for (int64_t i = 1; i < group; ++i) {
                if (x[i] < lo) lo = x[i];
                if (x[i] > hi) hi = x[i];
            }
            float range = hi - lo;
            if (range < 1e-9f) range = 1e-9f;
            float s = range / 15.0f;
            float z = lo + 8.0f * s;
            scale[r * ngroups + g] = s;
            zero[r * ngroups + g] = z;
            for (int64_t i = 0; i < group; ++i) {
                float q = rintf((x[i] - lo) / s);
                if (q < 0.0f) q = 0.0f;
                if (q > 15.0f) q = 15.0f;
                int64_t col = g * group + i;
                uint8_t *byte = &packed[r * (k / 2) + col / 2];
                uint8_t code = (uint8_t)q;
                if (col % 2 == 0) *byte = (uint8_t)((*byte & 0xF0u) | code);
                else *byte = (uint8_t)((*byte & 0x0Fu) | (code << 4));
            }
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Dequantization of one output channel (row n) to fp32.                    */
/* ---------------------------------------------------------------------- */

/* int4, groupwise: w = (q - 8) * scale[n, k/g] + zero[n, k/g]   [cpuint4]
 * docstring; groups along K [acext] 1.3.3.  Evaluated in fp32 as
 * CPUInt4EmbeddingMethod.embedding does: the product is exact, the add rounds.
 * group -1 (or >= k): one scale and zero per output channel (the per-column
 * mode of [acext] 1.3.2, which passes k as the group size).  zero == NULL:
 * scale-only, w = (q - 8) * scale, i.e. a zero of 0 ([acext] 1.3.2 runs
 * int4 with scales and no zero points; the unsigned code q stands for the
 * signed value q - 8). */
static void dequant4_row(const uint8_t *packed, const uint16_t *scale, const uint16_t *zero,
                         int64_t row, int64_t k, int64_t group, int dtype, float *w)
{
    int64_t ngroups = (group <= 0 || group >= k) ? 1 : k / group;
    int64_t gsz = (ngroups == 1) ? k : group;
    for (int64_t c = 0; c < k; ++c) {
        uint8_t byte = packed[row * (k / 2) + c / 2];
        int q = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        float s = act_to_f32(scale[row * ngroups + c / gsz], dtype);
        float z = zero ? act_to_f32(zero[row * ngroups + c / gsz], dtype) : 0.0f;
        float prod = (float)(q - 8) * s;
        w[c] = prod + z;
    }
}

/* int8 weight-only: one scale per output channel [acext] 1.3.1, group -1
 * [allspark]; with a group size g < K the scale is scale[n, k/g]. */
static void dequant8_row(const int8_t *codes, const uint16_t *scale, int64_t row, int64_t k,
                         int64_t group, int dtype, float *w)
{
    int64_t ngroups = (group <= 0 || group >= k) ? 1 : k / group;
    int64_t gsz = (ngroups == 1) ? k : group;
    for (int64_t c = 0; c < k; ++c) {
        float s = act_to_f32(scale[row * ngroups + c / gsz], dtype);
        w[c] = (float)codes[row * k + c] * s;
    }
}

void qref_dequant4(const uint8_t *packed, const uint16_t *scale, const uint16_t *zero,
                   int64_t n, int64_t k, int64_t group, int dtype, float *w_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) dequant4_row(packed, scale, zero, r, k, group, dtype, w_out + r * k);
}

void qref_dequant8(const int8_t *codes, const uint16_t *scale, int64_t n, int64_t k,
                   int64_t group, int dtype, float *w_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) dequant8_row(codes, scale, r, k, group, dtype, w_out + r * k);
}

/* ---------------------------------------------------------------------- */
/* Embedding lookup  [cpuint4] CPUInt4EmbeddingMethod.embedding: gather the */
/* rows of the quantized vocab table named by the token ids, dequantize     */
/* them in fp32 with the same rule as the linear layers (the table is the   */
/* tied output head), and hand them on in the activation dtype.  Here the   */
/* fp32 rows are written; rounding to the 16-bit dtype is qref_f32_to_*.    */
/* Ids outside [0, vocab) have no row in the page's definition; this oracle */
/* gives them a row of zeros.                                               */
/* ---------------------------------------------------------------------- */
void qref_embed4(const int32_t *ids, int64_t tokens, const uint8_t *packed, const uint16_t *scale,
                 const uint16_t *zero, int64_t vocab, int64_t hidden, int64_t group, int dtype,
                 float *out)
{
    for (int64_t t = 0; t < tokens; ++t) {
        float *o = out + t * hidden;
        if (ids[t] < 0 || ids[t] >= vocab) {
            for (int64_t c = 0; c < hidden; ++c) o[c] = 0.0f;
            continue;
        }
        dequant4_row(packed, scale, zero, ids[t], hidden, group, dtype, o);
    }
}

void qref_embed8(const int32_t *ids, int64_t tokens, const int8_t *codes, const uint16_t *scale,
                 int64_t vocab, int64_t hidden, int64_t group, int dtype, float *out)
{
    for (int64_t t = 0; t < tokens; ++t) {
        float *o = out + t * hidden;
        if (ids[t] < 0 || ids[t] >= vocab) {
            for (int64_t c = 0; c < hidden; ++c) o[c] = 0.0f;
            continue;
        }
        dequant8_row(codes, scale, ids[t], hidden, group, dtype, o);
    }
}

/* ---------------------------------------------------------------------- */
/* GEMM  C[m, n] = sum_k A[m, k] * W[n, k] (+ bias[n])   [acext] 1.2.1,    */
/* bias after the product [cpuint4] CPUInt4LinearMethod.apply.  Double      */
/* accumulation, result left unrounded in double.                           */
/* ---------------------------------------------------------------------- */

static double dot_row(const uint16_t *A, int64_t m, int64_t k, int dtype, const float *w)
{
    double acc = 0.0;
    for (int64_t c = 0; c < k; ++c) acc += act_to_double(A[m * k + c], dtype) * (double)w[c];
    return acc;
}

static double bias_value(const uint16_t *bias, int64_t col, int bias_dtype)
{
    if (!bias || bias_dtype == QREF_NONE) return 0.0;
    return act_to_double(bias[col], bias_dtype);
}

void qref_gemm_w4(const uint16_t *A, const uint8_t *packed, const uint16_t *scale,
                  const uint16_t *zero, const uint16_t *bias, int64_t m, int64_t n, int64_t k,
                  int64_t group, int dtype, int bias_dtype, double *C)
{
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 16)
        for (int64_t col = 0; col < n; ++col) {
            dequant4_row(packed, scale, zero, col, k, group, dtype, w);
            double b = bias_value(bias, col, bias_dtype);
            for (int64_t row = 0; row < m; ++row) C[row * n + col] = dot_row(A, row, k, dtype, w) + b;
        }
        free(w);
    }
}

void qref_gemm_w8(const uint16_t *A, const int8_t *codes, const uint16_t *scale,
                  const uint16_t *bias, int64_t m, int64_t n, int64_t k, int64_t group,
                  int dtype, int bias_dtype, double *C)
{
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 16)
        for (int64_t col = 0; col < n; ++col) {
            dequant8_row(codes, scale, col, k, group, dtype, w);
            double b = bias_value(bias, col, bias_dtype);
            for (int64_t row = 0; row < m; ++row) C[row * n + col] = dot_row(A, row, k, dtype, w) + b;
        }
        free(w);
    }
}

/* The same GEMMs with the sum carried in fp32 instead of double: each
 * product A[m, k] * W[n, k] rounds to fp32, then each add rounds (no fused
 * multiply-add: the library is built with contraction off), in k order, and
 * the bias is added last in fp32.  This is the plain fp32-accumulating CPU
 * GEMM whose speed the benchmark reports beside the GPU's; its results are
 * checked against the double-accumulating definition above (they agree to
 * fp32 rounding of a K-term sum). */
static float dot_row_f32(const uint16_t *A, int64_t m, int64_t k, int dtype, const float *w)
{
    float acc = 0.0f;
    for (int64_t c = 0; c < k; ++c) acc += act_to_f32(A[m * k + c], dtype) * w[c];
    return acc;
}

static float bias_value_f32(const uint16_t *bias, int64_t col, int bias_dtype)
{
    if (!bias || bias_dtype == QREF_NONE) return 0.0f;
    return act_to_f32(bias[col], bias_dtype);
}

void qref_gemm_w4_f32acc(const uint16_t *A, const uint8_t *packed, const uint16_t *scale,
                         const uint16_t *zero, const uint16_t *bias, int64_t m, int64_t n,
                         int64_t k, int64_t group, int dtype, int bias_dtype, float *C)
{
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 16)
        for (int64_t col = 0; col < n; ++col) {
            dequant4_row(packed, scale, zero, col, k, group, dtype, w);
            float b = bias_value_f32(bias, col, bias_dtype);
            for (int64_t row = 0; row < m; ++row) C[row * n + col] = dot_row_f32(A, row, k, dtype, w) + b;
        }
        free(w);
    }
}

void qref_gemm_w8_f32acc(const uint16_t *A, const int8_t *codes, const uint16_t *scale,
                         const uint16_t *bias, int64_t m, int64_t n, int64_t k, int64_t group,
                         int dtype, int bias_dtype, float *C)
{
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 16)
        for (int64_t col = 0; col < n; ++col) {
            dequant8_row(codes, scale, col, k, group, dtype, w);
            float b = bias_value_f32(bias, col, bias_dtype);
            for (int64_t row = 0; row < m; ++row) C[row * n + col] = dot_row_f32(A, row, k, dtype, w) + b;
        }
        free(w);
    }
}

/* The same definitions evaluated only at chosen (row, col) pairs, for
 * shapes whose full product is too large to compute on the CPU. */
void qref_gemm_w4_at(const uint16_t *A, const uint8_t *packed, const uint16_t *scale,
                     const uint16_t *zero, const uint16_t *bias, int64_t m, int64_t n, int64_t k,
                     int64_t group, int dtype, int bias_dtype, const int64_t *rows,
                     const int64_t *cols, int64_t count, double *out)
{
    (void)m; (void)n;
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < count; ++i) {
            dequant4_row(packed, scale, zero, cols[i], k, group, dtype, w);
            out[i] = dot_row(A, rows[i], k, dtype, w) + bias_value(bias, cols[i], bias_dtype);
        }
        free(w);
    }
}

void qref_gemm_w8_at(const uint16_t *A, const int8_t *codes, const uint16_t *scale,
                     const uint16_t *bias, int64_t m, int64_t n, int64_t k, int64_t group,
                     int dtype, int bias_dtype, const int64_t *rows, const int64_t *cols,
                     int64_t count, double *out)
{
    (void)m; (void)n;
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < count; ++i) {
            dequant8_row(codes, scale, cols[i], k, group, dtype, w);
            out[i] = dot_row(A, rows[i], k, dtype, w) + bias_value(bias, cols[i], bias_dtype);
        }
        free(w);
    }
}

/* ---------------------------------------------------------------------- */
/* W8A8: int8 activations times int8 weights  [acext] 1.2.2 w8a8 GEMM and   */
/* 1.3.4 SmoothQuant: C[m, n] = (sum_k A[m, k] B[n, k]) * alpha_row * alpha_col */
/* with alpha_row one value (per tensor) or one per row m (per token) and    */
/* alpha_col one value or one per output channel n; both fp32.  The integer */
/* sum is exact (int64); the scaling is done in double.                      */
/* ---------------------------------------------------------------------- */
void qref_gemm_w8a8(const int8_t *A, const int8_t *B, const float *alpha_row, int per_token,
                    const float *alpha_col, int per_channel, int64_t m, int64_t n, int64_t k,
                    int64_t *acc_out, double *C)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t col = 0; col < n; ++col) {
        for (int64_t row = 0; row < m; ++row) {
            int64_t acc = 0;
            for (int64_t c = 0; c < k; ++c) acc += (int64_t)A[row * k + c] * (int64_t)B[col * k + c];
            double ar = (double)alpha_row[per_token ? row : 0];
            double ac = (double)alpha_col[per_channel ? col : 0];
            if (acc_out) acc_out[row * n + col] = acc;
            C[row * n + col] = (double)acc * ar * ac;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* MoE  [acext] 1.2.3 runMoe: fp32 gating logits, top-k experts per row,   */
/* normalised expert scales, fc1 with a gated activation, fc2, and a        */
/* weighted combine into the final output.                                  */
/* ---------------------------------------------------------------------- */

/* Routing  [acext] 1.2.3 runMoe: fp32 gating logits, an optional second
 * set of logits "with bias" used to choose the experts, rows marked
 * finished, and the expert-scale normalization mode.
 * Selection: the topk largest selection logits (the biased set when given,
 * else the gating logits), descending, ties to the lower index.
 * Weights, from the unbiased gating logits l:
 *   renormalize: exp(l_e) / sum over the selected experts of exp(l)
 *   none:        exp(l_e) / sum over all experts of exp(l)  (the softmax
 *                probability, not renormalized)
 * both in double, shifted by the largest l of the sum for range.  A finished
 * row takes no expert: ids -1, weights 0. */
void qref_moe_route_ex(const float *logits, const float *sel_logits, const uint8_t *finished,
                       int64_t tokens, int64_t experts, int64_t topk, int renormalize,
                       int32_t *ids, double *weights)
{
    for (int64_t t = 0; t < tokens; ++t) {
        const float *l = logits + t * experts;
        const float *sl = sel_logits ? sel_logits + t * experts : l;
        if (finished && finished[t]) {
            for (int64_t j = 0; j < topk; ++j) { ids[t * topk + j] = -1; weights[t * topk + j] = 0.0; }
            continue;
        }
        for (int64_t j = 0; j < topk; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < experts; ++e) {
                int taken = 0;
                for (int64_t p = 0; p < j; ++p) if (ids[t * topk + p] == (int32_t)e) taken = 1;
                if (taken) continue;
                if (best < 0 || sl[e] > sl[best]) best = e;   /* strict: ties keep lower index */
            }
            ids[t * topk + j] = (int32_t)best;
        }
        double lmax = -INFINITY, denom = 0.0;
        if (renormalize) {
            for (int64_t j = 0; j < topk; ++j)
                if ((double)l[ids[t * topk + j]] > lmax) lmax = (double)l[ids[t * topk + j]];
            for (int64_t j = 0; j < topk; ++j) denom += exp((double)l[ids[t * topk + j]] - lmax);
        } else {
            for (int64_t e = 0; e < experts; ++e) if ((double)l[e] > lmax) lmax = (double)l[e];
            for (int64_t e = 0; e < experts; ++e) denom += exp((double)l[e] - lmax);
        }
        for (int64_t j = 0; j < topk; ++j)
            weights[t * topk + j] = exp((double)l[ids[t * topk + j]] - lmax) / denom;
    }
}

/* Top-k selection over raw logits, descending, ties to the lower index;
 * weights = softmax restricted to the selected logits (in double). */
void qref_moe_route(const float *logits, int64_t tokens, int64_t experts, int64_t topk,
                    int32_t *ids, double *weights)
{
    qref_moe_route_ex(logits, NULL, NULL, tokens, experts, topk, 1, ids, weights);
}

static double silu(double x) { return x / (1.0 + exp(-x)); }

/* out[t, :] = sum_j w[t, j] * fc2_e( silu(gate) * up ),  e = ids[t, j],
 * gate/up = rows [0, I) / [I, 2I) of fc1_e applied to x[t] (plus the fc1
 * bias b1[e] when given), fc2_e(a) = W2_e a (plus the fc2 bias b2[e]).
 * Weights of expert e: w1 packed [E][2I][H/2], s1/z1 [E][2I][H/g], w2 packed
 * [E][H][I/2], s2/z2 [E][H][I/g]; biases b1 [E][2I] and b2 [E][H] in the
 * activation dtype ([acext] 1.2.3 runMoe's fc1/fc2 expert biases).  Routing
 * as qref_moe_route_ex; finished rows get an output of zeros.  Only the
 * tokens listed in `sel` (count ntok) are computed; out is [ntok, H] in
 * double.  Expert-major so that each expert's weights are dequantized once. */
void qref_moe_ex(const uint16_t *x, const float *logits, const float *sel_logits,
                 const uint8_t *finished, const uint8_t *w1, const uint16_t *s1,
                 const uint16_t *z1, const uint16_t *b1, const uint8_t *w2, const uint16_t *s2,
                 const uint16_t *z2, const uint16_t *b2, int64_t tokens, int64_t hidden,
                 int64_t inter, int64_t experts, int64_t topk, int64_t group, int renormalize,
                 int dtype, const int64_t *sel, int64_t ntok, int32_t *ids_out,
                 double *weights_out, double *out)
{
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(tokens * topk));
    double *wts = (double *)malloc(sizeof(double) * (size_t)(tokens * topk));
    qref_moe_route_ex(logits, sel_logits, finished, tokens, experts, topk, renormalize, ids, wts);
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)(tokens * topk));
    if (weights_out) memcpy(weights_out, wts, sizeof(double) * (size_t)(tokens * topk));
    memset(out, 0, sizeof(double) * (size_t)(ntok * hidden));

    int64_t two_i = 2 * inter;
    float *W1 = (float *)malloc(sizeof(float) * (size_t)(two_i * hidden));
    float *W2 = (float *)malloc(sizeof(float) * (size_t)(hidden * inter));
    for (int64_t e = 0; e < experts; ++e) {
        const uint8_t *w1e = w1 + e * two_i * (hidden / 2);
        const uint16_t *s1e = s1 + e * two_i * (hidden / group);
        const uint16_t *z1e = z1 + e * two_i * (hidden / group);
        const uint8_t *w2e = w2 + e * hidden * (inter / 2);
        const uint16_t *s2e = s2 + e * hidden * (inter / group);
        const uint16_t *z2e = z2 + e * hidden * (inter / group);
        int used = 0;
        for (int64_t i = 0; i < ntok && !used; ++i)
            for (int64_t j = 0; j < topk; ++j) if (ids[sel[i] * topk + j] == (int32_t)e) used = 1;
        if (!used) continue;
        qref_dequant4(w1e, s1e, z1e, two_i, hidden, group, dtype, W1);
        qref_dequant4(w2e, s2e, z2e, hidden, inter, group, dtype, W2);
#pragma omp parallel
        {
            double *h = (double *)malloc(sizeof(double) * (size_t)two_i);
            double *a = (double *)malloc(sizeof(double) * (size_t)inter);
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < ntok; ++i) {
                int64_t t = sel[i];
                for (int64_t j = 0; j < topk; ++j) {
                    if (ids[t * topk + j] != (int32_t)e) continue;
                    for (int64_t r = 0; r < two_i; ++r) {
                        double acc = 0.0;
                        for (int64_t c = 0; c < hidden; ++c)
                            acc += act_to_double(x[t * hidden + c], dtype) * (double)W1[r * hidden + c];
                        if (b1) acc += act_to_double(b1[e * two_i + r], dtype);
                        h[r] = acc;
                    }
                    for (int64_t r = 0; r < inter; ++r) a[r] = silu(h[r]) * h[inter + r];
                    double wj = wts[t * topk + j];
                    for (int64_t r = 0; r < hidden; ++r) {
                        double acc = 0.0;
                        for (int64_t c = 0; c < inter; ++c) acc += a[c] * (double)W2[r * inter + c];
                        if (b2) acc += act_to_double(b2[e * hidden + r], dtype);
                        out[i * hidden + r] += wj * acc;
                    }
                }
            }
            free(h); free(a);
        }
    }
    free(W1); free(W2); free(ids); free(wts);
}

void qref_moe(const uint16_t *x, const float *logits, const uint8_t *w1, const uint16_t *s1,
              const uint16_t *z1, const uint8_t *w2, const uint16_t *s2, const uint16_t *z2,
              int64_t tokens, int64_t hidden, int64_t inter, int64_t experts, int64_t topk,
              int64_t group, int dtype, const int64_t *sel, int64_t ntok, int32_t *ids_out,
              double *weights_out, double *out)
{
    qref_moe_ex(x, logits, NULL, NULL, w1, s1, z1, NULL, w2, s2, z2, NULL, tokens, hidden, inter,
                experts, topk, group, 1, dtype, sel, ntok, ids_out, weights_out, out);
}
