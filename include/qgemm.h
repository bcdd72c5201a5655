/*
 * qgemm.h -- C ABI of the MI355X (gfx950) weight-only quantized GEMM library.
 *
 * The operation (fpA_intB): C[m, n] = sum_k A[m, k] * W[n, k] (+ bias[n]),
 * where A is a bf16/fp16 activation matrix and W is dequantized on the fly
 * from integer codes:
 *
 *   int4, groupwise:  W[n, k] = (q[n, k] - 8) * scale[n, k/g] + zero[n, k/g]
 *         (per channel with g = k; scale-only when there are no zeros:
 *         zero = 0, the scale-only forms of acext 1.3.2)
 *   int8, per channel: W[n, k] = q[n, k] * scale[n]
 *   int8, groupwise:   W[n, k] = q[n, k] * scale[n, k/g]   (no zero)
 *
 * Sources: "acext User Guide (v1.7)", 1.2.1 fpAintB GEMM (argument set: A,
 * B, scales, zero points, biases, C, m, n, k, group size, workspace, stream),
 * 1.3.1 Int8 Weight-only (one scale per output channel), 1.3.3 Int4
 * Groupwise (groups of 64 or 128, zero points for asymmetric grids), 1.2.3
 * MoE GEMM (runMoe); vllm-omni cpu_int4.py, module docstring (the portable
 * int4 checkpoint format and the dequant rule); "[Misc][Kernel]: Add
 * GPTQAllSpark Quantization", PR description (A16W8, group size -1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every buffer is owned by the caller.  Pointers marked "device" must be
 *    device memory on the current HIP device; the library allocates nothing
 *    and keeps no per-call state.
 *  - All matrices are dense row-major, contiguous, with no leading-dimension
 *    arguments.  Matrix pointers (A, codes, C, W, x, out) must be 16-byte
 *    aligned, vectors (scales, zeros, bias) 2-byte, fp32/int32 arrays
 *    4-byte, and a workspace 256-byte aligned.
 *  - 16-bit floats are passed as their raw storage (bf16 / IEEE binary16).
 *    scales and zeros always have the activation dtype; bias has its own.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; a QG_OK return means the launch was accepted.
 *  - Arguments are validated on the host before any HIP call.  On any error
 *    nothing is enqueued and the outputs are untouched.  m == 0 or n == 0 (or
 *    tokens == 0) is a successful no-op that reads no pointer; k must be
 *    positive (repack and dequant also accept k == 0).  The first failed
 *    check decides the status, in the order: sizes, NULL pointers, dtypes,
 *    mode arguments (W8A8 quant mode, table layout, MoE normalization), group
 *    size, tile multiples, alignment, workspace.
 *  - Functions are reentrant; calls on different streams may overlap unless
 *    they share a workspace.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_ERR_NULL = 1,        /* a required pointer is NULL */
    QG_ERR_SHAPE = 2,       /* negative size, or sizes that do not fit together */
    QG_ERR_GROUP = 3,       /* group size not supported, or k % group != 0 */
    QG_ERR_DTYPE = 4,       /* dtype code not allowed for this argument */
    QG_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned */
    QG_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
    QG_ERR_UNSUPPORTED = 7, /* valid, but outside the tile multiples listed per call */
    QG_ERR_HIP = 8,         /* the HIP runtime rejected a launch */
    QG_ERR_MODE = 9         /* a mode argument (W8A8 quant mode, table layout) outside its values */
} qg_status;

typedef enum { QG_NONE = 0, QG_BF16 = 1, QG_FP16 = 2, QG_FP32 = 3 } qg_dtype;

/* Human-readable name of a status code (static storage, never NULL).  The
 * pages give the GEMM runners no error channel ("acext User Guide (v1.7)",
 * 1.2.1: the runners return void); the explicit status follows the rule of
 * vllm-omni cpu_int4.py (supports_direct_dequant and the shape checks of
 * _create_int4_weights): refuse what is not supported, never misread it.
 * This function only names the codes. */
const char *qg_strerror(qg_status status);

/* Library version as 10000*major + 100*minor + patch.  No passage of the
 * pages applies (bookkeeping). */
int qg_version(void);

/* Dispatch override, for tests and tuning only (no passage of the pages
 * applies; no part of the method): forces choices the library otherwise
 * makes from a problem's sizes, for every later call in the process.
 * spec is a comma-separated list of key=value pairs:
 *   path=auto|decode|prefill        the GEMM path (else by m: decode for
 *                                   m <= 16)
 *   prefill_tile=auto|X|D8|D8N|D64|D128|L|M|S|P256|P128|P64|W256|W256N|W128|W64|WX
 *                                   the prefill tile (P: dequantize-then-
 *                                   dense, which needs n * k * 2 bytes of
 *                                   workspace; W: int8, codes converted
 *                                   after the LDS read; WX: 256 x 256 tiles
 *                                   and 128 x 128 quarters in one launch,
 *                                   forced: half the large tiles each)
 *   splitk=<n>                      prefill K slices (1: none), n >= 1
 *   moe_tile=auto|S                 S: the MoE on the 128 x 128 tile
 *   w8a8_tile=auto|T256|T256N|T128|T64   the W8A8 tile (also for m <= 16)
 *   w8a8_split=<n>                  W8A8 K slices, n >= 1
 * Keys not given take their automatic choice; NULL or "" restores every
 * automatic choice.  A forced choice that does not fit a problem (a
 * 256-wide tile for n % 256 != 0, the prefill path for n % 64 != 0) is
 * ignored for that problem.  The environment variable QGEMM_OVERRIDE, read
 * once when the library first dispatches, gives the initial spec (unless
 * this function was called before).  Returns QG_ERR_MODE, changing nothing,
 * for an unknown key or value.  Set it between calls: calls running on other
 * threads may see either setting. */
qg_status qg_set_override(const char *spec);

/* ------------------------------------------------------------------------
 * Load-side repack (once per weight).  The portable layouts are
 *   int4: uint8 [n, k/2], byte j of row n = q[n, 2j] | q[n, 2j+1] << 4
 *         (vllm-omni cpu_int4.py, module docstring);
 *   int8: int8 [n, k] row-major, signed two's complement.
 * The tiled layouts have the same byte count and are pure permutations
 * (int8 also flips the top bit), so the inverse recovers the input exactly.
 * Repacking once at load removes every per-call shuffle (the same reason
 * cpu_int4.py's to_split_halves de-interleaves nibbles once at load).
 *
 * int4 tiled layout (requires n % 16 == 0, k % 128 == 0): 1024-byte blocks,
 * one per (16 output channels) x (128 k).  For code q[n, k]:
 *     nt = n / 16, nl = n % 16, kb = k / 128, r = k % 128
 *     t = r / 32, j = (r / 8) % 4, e = k % 8
 *     lane = 16*j + nl
 *     pos  = (e even) ? e/2 : 4 + e/2           (nibble slot in a 32-bit word)
 *     byte = (nt*(k_total/128) + kb)*1024 + lane*16 + t*4 + pos/2
 *     nibble = pos % 2 (0 = low)
 * i.e. the 32-bit word (block, lane, t) holds the eight codes k = 128*kb +
 * 32*t + 8*j + 0..7 of channel n, even k in the low half-word.
 *
 * int8 tiled layout (requires n % 16 == 0, k % 64 == 0): 1024-byte blocks,
 * one per (16 channels) x (64 k).  For q[n, k]:
 *     nt = n / 16, nl = n % 16, kb = k / 64, r = k % 64
 *     t = r / 32, j = (r / 8) % 4, e = k % 8,  lane = 16*j + nl
 *     byte = (nt*(k_total/64) + kb)*1024 + lane*16 + t*8 + e
 *     stored value = (uint8)q ^ 0x80            (offset binary, q + 128)
 *
 * src and dst are device pointers and must not overlap.
 * ---------------------------------------------------------------------- */
qg_status qrepack_w4(const uint8_t *src_nk2, uint8_t *dst_tiled, int n, int k, void *stream);
qg_status qunrepack_w4(const uint8_t *src_tiled, uint8_t *dst_nk2, int n, int k, void *stream);
qg_status qrepack_w8(const int8_t *src_nk, int8_t *dst_tiled, int n, int k, void *stream);
qg_status qunrepack_w8(const int8_t *src_tiled, int8_t *dst_nk, int n, int k, void *stream);

/* int8 weights stored K-major: src_kn is int8 [k, n] row-major (the weight
 * orientation of "acext User Guide (v1.7)": 1.3.1 preprocesses a row-major
 * {k, n} weight, 2.1.2 allocates qweight as [input size, output size]).
 * qrepack_w8_kn writes the same tiled layout as qrepack_w8 of its [n, k]
 * transpose; qunrepack_w8_kn is its inverse (tiled -> [k, n]).  Same
 * requirements as qrepack_w8 (n % 16 == 0, k % 64 == 0, 16-byte aligned),
 * and k / 64 <= 65535. */
qg_status qrepack_w8_kn(const int8_t *src_kn, int8_t *dst_tiled, int n, int k, void *stream);
qg_status qunrepack_w8_kn(const int8_t *src_tiled, int8_t *dst_kn, int n, int k, void *stream);

/* ------------------------------------------------------------------------
 * Groupwise min/max 4-bit quantizer (vllm-omni cpu_int4.py,
 * quantize_groupwise): fp weights W [n, k] -> portable int4 codes and one
 * scale and zero per (row, K-group), chosen so that (q - 8) * scale + zero
 * gives the group's smallest value at q = 0 and its largest at q = 15.
 * For a group with smallest value lo and largest hi, all in fp32:
 *     scale = max(hi - lo, 1e-9) / 15
 *     zero  = lo + 8 * scale
 *     q     = round((w - lo) / scale), ties to even, clamped to [0, 15]
 * The division is the correctly rounded one, so the codes are bit-exact.
 *   W       device [n, k] in w_dtype (QG_BF16, QG_FP16 or QG_FP32)
 *   packed  device uint8 [n, k/2], the portable int4 layout above (pass it
 *           to qrepack_w4 before the GEMMs)
 *   scales, zeros  device [n, k/group] in sz_dtype: QG_FP32 (the values
 *           above) or QG_BF16 / QG_FP16 (those values rounded to nearest
 *           even, the form the GEMMs take; the codes still come from the
 *           fp32 scale)
 *   group_size: 64 or 128, k % group_size == 0.  n == 0 or k == 0: no-op.
 *   Alignment: W and packed 16 bytes; scales and zeros 4 bytes for fp32,
 *   else 2.  W must not overlap the outputs.
 * ---------------------------------------------------------------------- */
qg_status qquantize_w4(const void *W, uint8_t *packed, void *scales, void *zeros, int n, int k,
                       int group_size, qg_dtype w_dtype, qg_dtype sz_dtype, void *stream);

/* ------------------------------------------------------------------------
 * Dequantization hook (testing and fallback use): tiled codes -> W [n, k]
 * row-major in out_dtype (QG_FP32, or the activation dtype).  The rule is
 * vllm-omni cpu_int4.py's (module docstring: w = (q - 8) * scale + zero;
 * CPUInt4EmbeddingMethod.embedding: dequantize in fp32, then cast) and the
 * int8 rule of "acext User Guide (v1.7)" 1.3.1 (w = q * scale per channel).  The fp32
 * value is (q - 8) * s + z (int4; the product is exact, the add rounds to
 * nearest even) or q * s (int8, exact); the 16-bit output is that fp32 value
 * rounded to nearest even.  Bit-exact by contract.
 *   group_size: int4 64, 128 or -1 (= k, per channel); int8 -1 (per
 *   channel), 64 or 128.
 *   scales/zeros: [n, k/group] (groupwise) or [n] (per channel), act_dtype;
 *   zeros NULL (int4): scale-only, a zero of 0.
 * ---------------------------------------------------------------------- */
qg_status qdequant_w4(const uint8_t *B_tiled, const void *scales, const void *zeros, void *W_out,
                      int n, int k, int group_size, qg_dtype act_dtype, qg_dtype out_dtype,
                      void *stream);
qg_status qdequant_w8(const int8_t *B_tiled, const void *scales, void *W_out, int n, int k,
                      int group_size, qg_dtype act_dtype, qg_dtype out_dtype, void *stream);

/* ------------------------------------------------------------------------
 * GEMM.  (acext User Guide (v1.7), 1.2.1 fpAintB GEMM; 1.3.1; 1.3.3)
 *   A       device [m, k], act_dtype (QG_BF16 or QG_FP16)
 *   B_tiled device, the tiled layout above (qrepack_w4 / qrepack_w8 output)
 *   scales  device [n, k/group] (w4; w8 with group 64/128) or [n] (w8,
 *           group -1), act_dtype
 *   zeros   device [n, k/group], act_dtype (w4 only); NULL for scale-only
 *           int4 weights, w = (q - 8) * scale (acext 1.3.2 runs int4 with
 *           scales and no zero points)
 *   bias    device [n] in bias_dtype, or NULL with bias_dtype QG_NONE
 *   C       device [m, n], act_dtype; written, never read
 *   group_size: w4 64, 128, or -1 (one scale (and zero) per channel, [n];
 *           acext 1.3.2's per-column int4; k is accepted as a synonym);
 *           w8 -1 (k is accepted as a synonym of -1),
 *           64 or 128 (one scale per K-group; k % group_size == 0).  With
 *           groups the GEMMs stage q * s rounded to the activation dtype
 *           for the matrix cores (decode scales each block's fp32 partial
 *           product instead); per channel the scale multiplies the fp32 sum.
 *   Tile multiples: n % 16 == 0; k % 128 == 0 (w4) or k % 64 == 0 (w8);
 *   m is any value >= 0.  Accumulation is fp32; C = RNE(acc + bias).
 *   workspace: optional device scratch, 256-byte aligned.  When it holds at
 *   least qgemm_workspace_size() bytes (> 0 only for problems the prefill
 *   path splits along K -- today the 64 x 64 tile at m <= 128 with k >= 2048,
 *   and for int8 with one scale per channel the code-converting 64 x 128
 *   tile at m <= 128 when its tiles fill less than half the CUs -- or runs
 *   dequantize-then-dense) the K slices write fp32 partials
 *   [slices, m, n] there and one more launch sums them in slice order, then
 *   scales, adds bias and rounds; or the whole weight is dequantized there
 *   (n x k values in the activation type, vllm-omni cpu_int4.py: the int4
 *   linear's dequantize-then-dense path for batches of at least
 *   dequant_threshold rows) and one dense tile runs on it, bit-equal to the
 *   unsplit fused tiles.  With less (or NULL) the same call runs unsplit on
 *   the fused tiles.  Calls that share a workspace must not overlap.
 * ---------------------------------------------------------------------- */
size_t qgemm_workspace_size(int m, int n, int k, int group_size, int weight_bits);

qg_status qgemm_w4a16(const void *A, const uint8_t *B_tiled, const void *scales,
                      const void *zeros, const void *bias, void *C, int m, int n, int k,
                      int group_size, qg_dtype act_dtype, qg_dtype bias_dtype, void *workspace,
                      size_t workspace_bytes, void *stream);

qg_status qgemm_w8a16(const void *A, const int8_t *B_tiled, const void *scales, const void *bias,
                      void *C, int m, int n, int k, int group_size, qg_dtype act_dtype,
                      qg_dtype bias_dtype, void *workspace, size_t workspace_bytes,
                      void *stream);

/* ------------------------------------------------------------------------
 * W8A8: int8 activations times int8 weights with fp32 row and column scales
 * (acext User Guide (v1.7), 1.2.2 w8a8 GEMM: A, B, quant mode, alphaCol,
 * alphaRow, C, m, n, k, workspace, stream, the output type a parameter;
 * 1.3.4 SmoothQuant: both operands stay integer, four variants).
 *   C[m, n] = RNE_out( float(sum_k A[m, k] * B[n, k]) * alpha_row[r] * alpha_col[c] )
 * with the integer sum exact (int32), r = m for per-token activations (else
 * 0) and c = n for per-channel weights (else 0); the two fp32 products are
 * taken left to right.
 *   A          device int8 [m, k] row-major (activation codes)
 *   B          device int8 [n, k] row-major (weight codes, one row per output
 *              channel; no repack: the rows are already in the order the
 *              int8 matrix instruction reads)
 *   quant_mode QG_W8A8_PER_TENSOR (0), or an OR of QG_W8A8_PER_CHANNEL (1:
 *              alpha_col holds n values) and QG_W8A8_PER_TOKEN (2: alpha_row
 *              holds m values); the four values are the page's
 *              A_PerTensor_W_PerTensor, A_PerTensor_W_PerChannel,
 *              A_PerToken_W_PerTensor and A_PerToken_W_PerChannel
 *   alpha_col  device fp32 [n] (per channel) or [1]
 *   alpha_row  device fp32 [m] (per token) or [1]
 *   C          device [m, n] in out_dtype (QG_BF16, QG_FP16 or QG_FP32);
 *              written, never read
 *   Tile multiples: n % 16 == 0, k % 128 == 0, k <= 130944 (so that
 *   2^14 * k < 2^31: the int32 sum cannot overflow), m * k and n * k below
 *   2^31.  Alignment: A, B, C 16 bytes, alpha_* 4 bytes.
 *   workspace: optional, 256-byte aligned.  With at least
 *   qgemm_w8a8_workspace_size() bytes (> 0 when the output has too few tiles
 *   to fill the GPU, e.g. decode-sized m) K slices write int32 partials
 *   [slices, m, n] there and one more launch adds them (exactly) and scales;
 *   with less (or NULL) the same call runs unsplit.  Calls that share a
 *   workspace must not overlap.
 * ---------------------------------------------------------------------- */
enum { QG_W8A8_PER_TENSOR = 0, QG_W8A8_PER_CHANNEL = 1, QG_W8A8_PER_TOKEN = 2 };

size_t qgemm_w8a8_workspace_size(int m, int n, int k);

qg_status qgemm_w8a8(const int8_t *A, const int8_t *B, int quant_mode, const float *alpha_col,
                     const float *alpha_row, void *C, int m, int n, int k, qg_dtype out_dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Quantized embedding lookup (vllm-omni cpu_int4.py, CPUInt4EmbeddingMethod:
 * with tied embeddings the vocab table is the quantized output head; a lookup
 * gathers the token's row, dequantizes it in fp32 with the linear layers'
 * rule and casts it to the activation dtype).
 *   out[t, :] = RNE_out( dequant(table)[ids[t], :] ),  a row of zeros when
 *   ids[t] is outside [0, vocab)
 * with the fp32 values of qdequant_w4 / qdequant_w8 (bit-exact by contract).
 *   ids     device int32 [tokens]
 *   table   device codes of the [vocab, hidden] table in `layout`:
 *           QG_LAYOUT_TILED (1), the qrepack_w4 / qrepack_w8 output that
 *           qgemm_w4a16 / qgemm_w8a16 read as the lm_head weight (one copy
 *           serves both), or QG_LAYOUT_PORTABLE (0), the portable layout
 *   scales, zeros  as for the GEMM of the same table (zeros optional, int4)
 *   out     device [tokens, hidden] in out_dtype (QG_FP32 or act_dtype)
 *   group_size: int4 64, 128, -1 (= hidden); int8 -1 (= hidden), 64, 128.
 *   Requires vocab >= 1, hidden % 8 == 0, and for the tiled layout the
 *   repack's multiples (vocab % 16, hidden % 128 for int4 or % 64 for int8).
 *   Alignment: ids 4 bytes, table and out 16, scales and zeros 2.
 * ---------------------------------------------------------------------- */
enum { QG_LAYOUT_PORTABLE = 0, QG_LAYOUT_TILED = 1 };

qg_status qembed_w4(const int32_t *ids, int tokens, const uint8_t *table, int layout,
                    const void *scales, const void *zeros, void *out, int vocab, int hidden,
                    int group_size, qg_dtype act_dtype, qg_dtype out_dtype, void *stream);
qg_status qembed_w8(const int32_t *ids, int tokens, const int8_t *table, int layout,
                    const void *scales, void *out, int vocab, int hidden, int group_size,
                    qg_dtype act_dtype, qg_dtype out_dtype, void *stream);

/* ------------------------------------------------------------------------
 * Top-k MoE with SiLU-gated int4 experts  (acext User Guide (v1.7), 1.2.3
 * MoE GEMM: fp32 gating logits, fc1 with a gated activation, fc2, expert
 * scales, routing maps, final output).
 *   x        device [tokens, hidden], act_dtype (QG_BF16 or QG_FP16)
 *   logits   device fp32 [tokens, experts]
 *   w1_tiled device, experts consecutive tiled int4 matrices [2*inter, hidden]:
 *            rows [0, inter) are the gate projection, [inter, 2*inter) up
 *   s1, z1   device [experts, 2*inter, hidden/group], act_dtype
 *   w2_tiled device, experts consecutive tiled int4 matrices [hidden, inter]
 *   s2, z2   device [experts, hidden, inter/group], act_dtype
 *   out      device [tokens, hidden], act_dtype
 *   topk_ids_out  optional device int32 [tokens, topk] (NULL to skip)
 *   topk_w_out    optional device fp32 [tokens, topk] (NULL to skip)
 * Routing: the topk largest logits per row, in descending order, ties to
 * the lower expert id (-0.0 equals 0.0; a NaN ranks above +inf, or below
 * -inf when its sign bit is set); weights = softmax over the selected
 * logits only.
 * out[t] = sum_j w[t, j] * fc2_e(silu(gate) * up), e = ids[t, j],
 * silu(x) = x / (1 + exp(-x)); the activation is rounded to act_dtype before
 * fc2, the combine sums in fp32 in rank order.
 * Requires hidden % 128 == 0, inter % 128 == 0, 1 <= topk <= experts <= 256,
 * topk <= 64, group_size 64 or 128.  workspace: at least
 * qmoe_workspace_size() bytes, 256-byte aligned; it holds the routing maps,
 * the tile list and the fc1/fc2 intermediates, and is overwritten.
 * ---------------------------------------------------------------------- */
size_t qmoe_workspace_size(int tokens, int hidden, int inter, int experts, int topk);

qg_status qmoe_grouped(const void *x, const float *logits, const uint8_t *w1_tiled,
                       const void *s1, const void *z1, const uint8_t *w2_tiled, const void *s2,
                       const void *z2, void *out, int tokens, int hidden, int inter, int experts,
                       int topk, int group_size, qg_dtype act_dtype, int32_t *topk_ids_out,
                       float *topk_w_out, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Allocation-free variant of qmoe_grouped, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, arguments and
 * results, with no workspace argument.  Its workspace is a 64 MiB device
 * array inside the library (one per GPU the library runs on, held until the
 * process ends; its address is looked up once per device on the first call
 * there); the call allocates nothing.  A problem whose qmoe_workspace_size()
 * exceeds 64 MiB (2^26 bytes; e.g. more than about 1600 tokens at hidden
 * 2048, inter 1408, 64 experts, top-6) returns QG_ERR_WORKSPACE before any
 * launch.  Every call on one GPU shares that array: calls that overlap on
 * one GPU (other streams, other threads) race and must be serialized by the
 * caller.  Nothing in the array needs clearing between calls. */
qg_status qmoe_grouped_noalloc(const void *x, const float *logits, const uint8_t *w1_tiled,
                               const void *s1, const void *z1, const uint8_t *w2_tiled,
                               const void *s2, const void *z2, void *out, int tokens, int hidden,
                               int inter, int experts, int topk, int group_size,
                               qg_dtype act_dtype, int32_t *topk_ids_out, float *topk_w_out,
                               void *stream);

/* The same MoE with the optional inputs of runMoe (acext User Guide (v1.7),
 * 1.2.3: gating_output_with_bias, fc1/fc2 expert biases, finished,
 * normalization_mode):
 *   sel_logits  optional device fp32 [tokens, experts]: the biased logits
 *               that choose the experts (NULL: the gating logits).  The
 *               weights always come from `logits`.
 *   finished    optional device uint8 [tokens] (bool): a nonzero row takes
 *               no expert (topk ids -1, weights 0) and its output row is 0.
 *   b1          optional device [experts, 2*inter], act_dtype: fc1 biases,
 *               added to gate and up before the activation.
 *   b2          optional device [experts, hidden], act_dtype: fc2 biases,
 *               added to each expert's output (in fp32, in the combine).
 *   norm_mode   QG_MOE_RENORMALIZE (1): softmax over the selected logits (as
 *               qmoe_grouped); QG_MOE_NORM_NONE (0): the full softmax
 *               probability of each selected expert, not renormalized.
 * The page's active_rows (the count of unfinished rows) follows from
 * `finished` and is not an argument.  Other arguments and requirements as
 * qmoe_grouped (the same workspace size); alignment: sel_logits 4 bytes,
 * b1 and b2 16 bytes. */
enum { QG_MOE_NORM_NONE = 0, QG_MOE_RENORMALIZE = 1 };

qg_status qmoe_grouped_ex(const void *x, const float *logits, const float *sel_logits,
                          const uint8_t *finished, const uint8_t *w1_tiled, const void *s1,
                          const void *z1, const void *b1, const uint8_t *w2_tiled, const void *s2,
                          const void *z2, const void *b2, void *out, int tokens, int hidden,
                          int inter, int experts, int topk, int group_size, int norm_mode,
                          qg_dtype act_dtype, int32_t *topk_ids_out, float *topk_w_out,
                          void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Measurement probe (no part of the method): the ceiling the HBM-bound
 * kernels are compared with.  Reads `bytes` (a multiple of 16) of `buf` once
 * with 16-byte streaming loads, the grid sweeping one contiguous window, and
 * writes one 32-bit XOR of what it read per workgroup to `out` (device, at
 * least qg_read_probe_blocks(bytes) entries).  bytes == 0 launches one
 * workgroup that reads nothing: the cost of a launch.  buf 16-byte aligned
 * (may be NULL when bytes == 0), out 4-byte aligned.
 * ---------------------------------------------------------------------- */
size_t qg_read_probe_blocks(size_t bytes);
qg_status qg_read_probe(const void *buf, size_t bytes, uint32_t *out, void *stream);

/* LDS read probe (a measurement; no part of the method): `blocks`
 * workgroups of 64 * waves threads (waves 4, 8 or 16), each holding 96 KiB
 * of LDS so that no two share a CU, read their LDS with conflict-free 16-byte
 * loads, `iters` per thread, and write the shader-clock cycles of that loop
 * to cycles[b] (device, `blocks` entries, 8-byte aligned).  LDS bytes per
 * clock per CU = iters * waves * 64 * 16 / cycles[b].  Errors: QG_ERR_SHAPE
 * (blocks outside 1..65536, iters outside 8..2^20 or not a multiple of 8),
 * QG_ERR_MODE (waves), QG_ERR_NULL, QG_ERR_ALIGN. */
qg_status qg_lds_probe(int waves, int iters, int blocks, unsigned long long *cycles, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
