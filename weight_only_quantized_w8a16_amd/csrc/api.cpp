// api.cpp -- the C ABI of libqgemm (include/qgemm.h): host-side validation,
// path selection and launch.  Nothing here touches the GPU before every
// argument has been checked; on error nothing is enqueued.
#include <hip/hip_runtime.h>

#include "../../include/qgemm.h"
#include "qg_launch.hpp"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool act_ok(qg_dtype d) { return d == QG_BF16 || d == QG_FP16; }
hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }
qg_status hip_status(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ERR_HIP; }

constexpr int kDecodeMaxM = 16;

// Rows [m0, m0 + 16) at a time through the decode kernels.
template <class F>
hipError_t by_row_slabs(const qg::GemmArgs &a, F launch, hipStream_t s) {
  const int N = a.N, K = a.K;
  for (int m0 = 0; m0 < a.M; m0 += kDecodeMaxM) {
    qg::GemmArgs b = a;
    b.A = a.A + static_cast<size_t>(m0) * K;
    b.C = a.C + static_cast<size_t>(m0) * N;
    b.M = a.M - m0 < kDecodeMaxM ? a.M - m0 : kDecodeMaxM;
    hipError_t e = launch(b, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Checks in the documented order: sizes, NULL, dtypes, group, tile
// multiples, alignment.
qg_status gemm_checks(const void *A, const void *B, const void *scales, const void *zeros,
                      const void *C, const void *bias, int m, int n, int k, int group,
                      qg_dtype act, qg_dtype bias_dt, int wbits) {
  if (m < 0 || n < 0 || k <= 0) return QG_ERR_SHAPE;
  if (m == 0 || n == 0) return QG_OK;   // nothing to compute; pointers unused
  if (!A || !B || !scales || !C) return QG_ERR_NULL;   // zeros are optional (int4)
  if (bias_dt != QG_NONE && !bias) return QG_ERR_NULL;
  if (!act_ok(act)) return QG_ERR_DTYPE;
  if (bias_dt == QG_NONE ? bias != nullptr : !act_ok(bias_dt)) return QG_ERR_DTYPE;
  if (wbits == 4) {
    if (group != 64 && group != 128 && group != -1 && group != k) return QG_ERR_GROUP;
    if (group > 0 && k % group != 0) return QG_ERR_GROUP;
    if (n % 16 != 0 || k % 128 != 0) return QG_ERR_UNSUPPORTED;
  } else {
    if (group != -1 && group != k && group != 64 && group != 128) return QG_ERR_GROUP;
    if (group > 0 && k % group != 0) return QG_ERR_GROUP;
    if (n % 16 != 0 || k % 64 != 0) return QG_ERR_UNSUPPORTED;
  }
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(scales, 2) ||
      (zeros && !aligned(zeros, 2)) || (bias && !aligned(bias, 2)))
    return QG_ERR_ALIGN;
  return QG_OK;
}

}  // namespace

extern "C" {

const char *qg_strerror(qg_status s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "a required pointer is NULL";
    case QG_ERR_SHAPE: return "invalid or inconsistent sizes";
    case QG_ERR_GROUP: return "unsupported group size, or k is not a multiple of it";
    case QG_ERR_DTYPE: return "dtype not allowed for this argument";
    case QG_ERR_ALIGN: return "pointer not aligned (16 bytes for matrices, 2 for vectors)";
    case QG_ERR_WORKSPACE: return "workspace missing or too small";
    case QG_ERR_UNSUPPORTED: return "sizes outside the supported tile multiples";
    case QG_ERR_HIP: return "HIP runtime error at launch";
    case QG_ERR_MODE: return "mode argument (W8A8 quant mode, table layout) outside its values";
  }
  return "unknown status";
}

int qg_version(void) { return kVersion; }

// ---------------------------------------------------------------------------
// Repack
// ---------------------------------------------------------------------------
static qg_status repack_checks(const void *src, const void *dst, int n, int k, int kmul) {
  if (n < 0 || k < 0) return QG_ERR_SHAPE;
  if (n == 0 || k == 0) return QG_OK;
  if (!src || !dst) return QG_ERR_NULL;
  if (n % 16 != 0 || k % kmul != 0) return QG_ERR_UNSUPPORTED;
  if (!aligned(src, 16) || !aligned(dst, 16)) return QG_ERR_ALIGN;
  return QG_OK;
}

qg_status qrepack_w4(const uint8_t *src, uint8_t *dst, int n, int k, void *stream) {
  qg_status st = repack_checks(src, dst, n, k, 128);
  if (st != QG_OK || n == 0 || k == 0) return st;
  return hip_status(qg::launch_repack_w4(src, dst, n, k, as_stream(stream)));
}
qg_status qunrepack_w4(const uint8_t *src, uint8_t *dst, int n, int k, void *stream) {
  qg_status st = repack_checks(src, dst, n, k, 128);
  if (st != QG_OK || n == 0 || k == 0) return st;
  return hip_status(qg::launch_unrepack_w4(src, dst, n, k, as_stream(stream)));
}
qg_status qrepack_w8(const int8_t *src, int8_t *dst, int n, int k, void *stream) {
  qg_status st = repack_checks(src, dst, n, k, 64);
  if (st != QG_OK || n == 0 || k == 0) return st;
  return hip_status(qg::launch_repack_w8(src, dst, n, k, as_stream(stream)));
}
qg_status qunrepack_w8(const int8_t *src, int8_t *dst, int n, int k, void *stream) {
  qg_status st = repack_checks(src, dst, n, k, 64);
  if (st != QG_OK || n == 0 || k == 0) return st;
  return hip_status(qg::launch_unrepack_w8(src, dst, n, k, as_stream(stream)));
}
qg_status qrepack_w8_kn(const int8_t *src, int8_t *dst, int n, int k, void *stream) {
  qg_status st = repack_checks(src, dst, n, k, 64);
  if (st != QG_OK || n == 0 || k == 0) return st;
  if (static_cast<long long>(k / 64) > 65535) return QG_ERR_UNSUPPORTED;
  return hip_status(qg::launch_repack_w8_kn(src, dst, n, k, as_stream(stream)));
}
qg_status qunrepack_w8_kn(const int8_t *src, int8_t *dst, int n, int k, void *stream) {
  qg_status st = repack_checks(src, dst, n, k, 64);
  if (st != QG_OK || n == 0 || k == 0) return st;
  if (static_cast<long long>(k / 64) > 65535) return QG_ERR_UNSUPPORTED;
  return hip_status(qg::launch_unrepack_w8_kn(src, dst, n, k, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// Quantizer
// ---------------------------------------------------------------------------
qg_status qquantize_w4(const void *W, uint8_t *packed, void *scales, void *zeros, int n, int k,
                       int group, qg_dtype w_dt, qg_dtype sz_dt, void *stream) {
  if (n < 0 || k < 0) return QG_ERR_SHAPE;
  if (n == 0 || k == 0) return QG_OK;
  if (!W || !packed || !scales || !zeros) return QG_ERR_NULL;
  if (!(act_ok(w_dt) || w_dt == QG_FP32) || !(act_ok(sz_dt) || sz_dt == QG_FP32))
    return QG_ERR_DTYPE;
  if (group != 64 && group != 128) return QG_ERR_GROUP;
  if (k % group != 0) return QG_ERR_GROUP;
  const size_t sz_align = sz_dt == QG_FP32 ? 4 : 2;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, sz_align) ||
      !aligned(zeros, sz_align))
    return QG_ERR_ALIGN;
  return hip_status(qg::launch_quantize_w4(W, packed, scales, zeros, n, k, group,
                                           static_cast<int>(w_dt), static_cast<int>(sz_dt),
                                           as_stream(stream)));
}

// ---------------------------------------------------------------------------
// Dequant hook
// ---------------------------------------------------------------------------
qg_status qdequant_w4(const uint8_t *B, const void *scales, const void *zeros, void *W, int n,
                      int k, int group, qg_dtype act, qg_dtype out, void *stream) {
  if (n < 0 || k < 0) return QG_ERR_SHAPE;
  if (n == 0 || k == 0) return QG_OK;
  if (!B || !scales || !W) return QG_ERR_NULL;   // zeros optional
  if (!act_ok(act) || !(out == QG_FP32 || out == act)) return QG_ERR_DTYPE;
  if (group != 64 && group != 128 && group != -1 && group != k) return QG_ERR_GROUP;
  if (group > 0 && k % group != 0) return QG_ERR_GROUP;
  if (n % 16 != 0 || k % 128 != 0) return QG_ERR_UNSUPPORTED;
  if (!aligned(B, 16) || !aligned(W, 16) || !aligned(scales, 2) || (zeros && !aligned(zeros, 2)))
    return QG_ERR_ALIGN;
  return hip_status(qg::launch_dequant_w4(B, static_cast<const uint16_t *>(scales),
                                          static_cast<const uint16_t *>(zeros), W, n, k,
                                          group == -1 ? k : group, act, out, as_stream(stream)));
}

qg_status qdequant_w8(const int8_t *B, const void *scales, void *W, int n, int k, int group,
                      qg_dtype act, qg_dtype out, void *stream) {
  if (n < 0 || k < 0) return QG_ERR_SHAPE;
  if (n == 0 || k == 0) return QG_OK;
  if (!B || !scales || !W) return QG_ERR_NULL;
  if (!act_ok(act) || !(out == QG_FP32 || out == act)) return QG_ERR_DTYPE;
  if (group != -1 && group != k && group != 64 && group != 128) return QG_ERR_GROUP;
  if (group > 0 && k % group != 0) return QG_ERR_GROUP;
  if (n % 16 != 0 || k % 64 != 0) return QG_ERR_UNSUPPORTED;
  if (!aligned(B, 16) || !aligned(W, 16) || !aligned(scales, 2)) return QG_ERR_ALIGN;
  const int g = (group == -1 || group == k) ? 0 : group;
  return hip_status(qg::launch_dequant_w8(B, static_cast<const uint16_t *>(scales), W, n, k, g,
                                          act, out, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------
// Whether a GEMM runs on the prefill path (else the decode kernels).
// The dispatch override (qg_set_override) can force either path, so that
// tests can run both on the same inputs.
static bool uses_prefill(int m, int n) {
  const int f = qg::dispatch_override().path;
  const bool prefill_ok = n % 64 == 0;
  if (f == qg::kPathPrefill && prefill_ok) return true;
  return !(f == qg::kPathDecode || m <= kDecodeMaxM || !prefill_ok);
}

// Workspace: the prefill path's split-K partials for problems it would
// split; 0 for everything else (and for arguments a GEMM would reject).
size_t qgemm_workspace_size(int m, int n, int k, int group_size, int weight_bits) {
  if (m <= 0 || n <= 0 || k <= 0 || (weight_bits != 4 && weight_bits != 8)) return 0;
  if (!uses_prefill(m, n)) return 0;
  qg::GemmArgs a{};
  a.M = m;
  a.N = n;
  a.K = k;
  if (weight_bits == 4) a.group = group_size == -1 ? k : group_size;
  else a.group = (group_size == -1 || group_size == k) ? 0 : group_size;
  if (a.group < 0 || (a.group > 0 && k % a.group != 0)) return 0;
  const size_t b = qg::prefill_workspace_bytes(a, weight_bits);
  return b ? (b + 255) & ~static_cast<size_t>(255) : 0;
}

qg_status qgemm_w4a16(const void *A, const uint8_t *B, const void *scales, const void *zeros,
                      const void *bias, void *C, int m, int n, int k, int group, qg_dtype act,
                      qg_dtype bias_dt, void *workspace, size_t ws_bytes, void *stream) {
  qg_status st = gemm_checks(A, B, scales, zeros, C, bias, m, n, k, group, act, bias_dt, 4);
  if (st != QG_OK || m == 0 || n == 0) return st;
  if (workspace && ws_bytes && !aligned(workspace, 256)) return QG_ERR_ALIGN;
  qg::GemmArgs a{static_cast<const uint16_t *>(A), B, static_cast<const uint16_t *>(scales),
                 static_cast<const uint16_t *>(zeros), static_cast<const uint16_t *>(bias),
                 static_cast<uint16_t *>(C), m, n, k, group == -1 ? k : group,
                 static_cast<int>(act), static_cast<int>(bias_dt), workspace,
                 workspace ? ws_bytes : 0};
  hipStream_t s = as_stream(stream);
  if (uses_prefill(m, n)) return hip_status(qg::launch_prefill_w4(a, s));
  return hip_status(by_row_slabs(a, qg::launch_decode_w4, s));
}

qg_status qgemm_w8a16(const void *A, const int8_t *B, const void *scales, const void *bias,
                      void *C, int m, int n, int k, int group, qg_dtype act, qg_dtype bias_dt,
                      void *workspace, size_t ws_bytes, void *stream) {
  qg_status st = gemm_checks(A, B, scales, nullptr, C, bias, m, n, k, group, act, bias_dt, 8);
  if (st != QG_OK || m == 0 || n == 0) return st;
  if (workspace && ws_bytes && !aligned(workspace, 256)) return QG_ERR_ALIGN;
  const int g = (group == -1 || group == k) ? 0 : group;   // 0: one scale per channel
  qg::GemmArgs a{static_cast<const uint16_t *>(A), B, static_cast<const uint16_t *>(scales),
                 nullptr, static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(C),
                 m, n, k, g, static_cast<int>(act), static_cast<int>(bias_dt), workspace,
                 workspace ? ws_bytes : 0};
  hipStream_t s = as_stream(stream);
  if (uses_prefill(m, n)) return hip_status(qg::launch_prefill_w8(a, s));
  return hip_status(by_row_slabs(a, qg::launch_decode_w8, s));
}

// ---------------------------------------------------------------------------
// W8A8
// ---------------------------------------------------------------------------
// Largest k whose int32 sum cannot overflow (2^14 k < 2^31), rounded down to
// the 128-k step.
constexpr int kW8A8MaxK = 130944;

size_t qgemm_w8a8_workspace_size(int m, int n, int k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 128 != 0 || k > kW8A8MaxK) return 0;
  const size_t b = qg::w8a8_workspace_bytes(m, n, k);
  return b ? (b + 255) & ~static_cast<size_t>(255) : 0;
}

qg_status qgemm_w8a8(const int8_t *A, const int8_t *B, int mode, const float *alpha_col,
                     const float *alpha_row, void *C, int m, int n, int k, qg_dtype out,
                     void *workspace, size_t ws_bytes, void *stream) {
  if (m < 0 || n < 0 || k <= 0) return QG_ERR_SHAPE;
  if (m == 0 || n == 0) return QG_OK;   // nothing to compute; pointers unused
  if (!A || !B || !alpha_col || !alpha_row || !C) return QG_ERR_NULL;
  if (!(act_ok(out) || out == QG_FP32)) return QG_ERR_DTYPE;
  if (mode < 0 || mode > (QG_W8A8_PER_CHANNEL | QG_W8A8_PER_TOKEN)) return QG_ERR_MODE;
  const uint64_t lim = uint64_t(1) << 31;
  if (n % 16 != 0 || k % 128 != 0 || k > kW8A8MaxK || uint64_t(m) * k >= lim ||
      uint64_t(n) * k >= lim)
    return QG_ERR_UNSUPPORTED;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(alpha_col, 4) ||
      !aligned(alpha_row, 4))
    return QG_ERR_ALIGN;
  if (workspace && ws_bytes && !aligned(workspace, 256)) return QG_ERR_ALIGN;
  qg::W8A8Args a{A, B, alpha_row, alpha_col, C, m, n, k,
                 (mode & QG_W8A8_PER_TOKEN) ? 1 : 0, (mode & QG_W8A8_PER_CHANNEL) ? 1 : 0,
                 static_cast<int>(out), workspace, workspace ? ws_bytes : 0};
  return hip_status(qg::launch_w8a8(a, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// Embedding lookup
// ---------------------------------------------------------------------------
static qg_status embed(const int32_t *ids, int tokens, const void *table, int layout,
                       const void *scales, const void *zeros, void *out, int vocab, int hidden,
                       int group, qg_dtype act, qg_dtype out_dt, int bits, void *stream) {
  if (tokens < 0 || vocab <= 0 || hidden <= 0) return QG_ERR_SHAPE;
  if (tokens == 0) return QG_OK;   // nothing to look up; pointers unused
  if (!ids || !table || !scales || !out) return QG_ERR_NULL;   // zeros optional (int4)
  if (!act_ok(act) || !(out_dt == QG_FP32 || out_dt == act)) return QG_ERR_DTYPE;
  if (layout != QG_LAYOUT_PORTABLE && layout != QG_LAYOUT_TILED) return QG_ERR_MODE;
  if (group != 64 && group != 128 && group != -1 && group != hidden) return QG_ERR_GROUP;
  if (group > 0 && hidden % group != 0) return QG_ERR_GROUP;
  if (hidden % 8 != 0) return QG_ERR_UNSUPPORTED;
  if (layout == QG_LAYOUT_TILED && (vocab % 16 != 0 || hidden % (bits == 4 ? 128 : 64) != 0))
    return QG_ERR_UNSUPPORTED;
  if (!aligned(ids, 4) || !aligned(table, 16) || !aligned(out, 16) || !aligned(scales, 2) ||
      (zeros && !aligned(zeros, 2)))
    return QG_ERR_ALIGN;
  int g = group == -1 ? hidden : group;
  if (bits == 8 && g == hidden) g = 0;   // one scale per row
  qg::EmbedArgs a{ids, tokens, table, layout == QG_LAYOUT_TILED ? 1 : 0, bits,
                  static_cast<const uint16_t *>(scales), static_cast<const uint16_t *>(zeros), out,
                  vocab, hidden, g, static_cast<int>(act), static_cast<int>(out_dt)};
  return hip_status(qg::launch_embed(a, as_stream(stream)));
}

qg_status qembed_w4(const int32_t *ids, int tokens, const uint8_t *table, int layout,
                    const void *scales, const void *zeros, void *out, int vocab, int hidden,
                    int group, qg_dtype act, qg_dtype out_dt, void *stream) {
  return embed(ids, tokens, table, layout, scales, zeros, out, vocab, hidden, group, act, out_dt, 4,
               stream);
}

qg_status qembed_w8(const int32_t *ids, int tokens, const int8_t *table, int layout,
                    const void *scales, void *out, int vocab, int hidden, int group, qg_dtype act,
                    qg_dtype out_dt, void *stream) {
  return embed(ids, tokens, table, layout, scales, nullptr, out, vocab, hidden, group, act, out_dt, 8,
               stream);
}

// ---------------------------------------------------------------------------
// MoE
// ---------------------------------------------------------------------------
size_t qmoe_workspace_size(int tokens, int hidden, int inter, int experts, int topk) {
  if (tokens <= 0 || hidden <= 0 || inter <= 0 || experts <= 0 || topk <= 0) return 0;
  return qg::moe_workspace_bytes(tokens, hidden, inter, experts, topk);
}

static qg_status moe_call(const void *x, const float *logits, const float *sel_logits,
                          const uint8_t *finished, const uint8_t *w1, const void *s1,
                          const void *z1, const void *b1, const uint8_t *w2, const void *s2,
                          const void *z2, const void *b2, void *out, int tokens, int hidden,
                          int inter, int experts, int topk, int group, int norm, qg_dtype act,
                          int32_t *ids_out, float *w_out, void *workspace, size_t ws_bytes,
                          void *stream, bool noalloc = false) {
  if (tokens < 0 || hidden <= 0 || inter <= 0 || experts <= 0 || topk <= 0 || topk > experts)
    return QG_ERR_SHAPE;
  if (tokens == 0) return QG_OK;        // nothing to compute; pointers unused
  if (!x || !logits || !w1 || !s1 || !z1 || !w2 || !s2 || !z2 || !out) return QG_ERR_NULL;
  if (!act_ok(act)) return QG_ERR_DTYPE;
  if (norm != QG_MOE_NORM_NONE && norm != QG_MOE_RENORMALIZE) return QG_ERR_MODE;
  if (group != 64 && group != 128) return QG_ERR_GROUP;
  if (hidden % group != 0 || inter % group != 0) return QG_ERR_GROUP;
  if (hidden % 128 != 0 || inter % 128 != 0 || experts > 256 || topk > 64)
    return QG_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(logits, 4) || !aligned(s1, 2) || !aligned(z1, 2) || !aligned(s2, 2) ||
      !aligned(z2, 2) || (ids_out && !aligned(ids_out, 4)) || (w_out && !aligned(w_out, 4)) ||
      (sel_logits && !aligned(sel_logits, 4)) || (b1 && !aligned(b1, 16)) ||
      (b2 && !aligned(b2, 16)))
    return QG_ERR_ALIGN;
  const size_t need = qg::moe_workspace_bytes(tokens, hidden, inter, experts, topk);
  if (noalloc) {
    if (need > qg::kMoeScratchBytes) return QG_ERR_WORKSPACE;
  } else {
    if (!workspace || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QG_ERR_ALIGN;
  }
  qg::MoeArgs a{static_cast<const uint16_t *>(x), logits, w1,
                static_cast<const uint16_t *>(s1), static_cast<const uint16_t *>(z1), w2,
                static_cast<const uint16_t *>(s2), static_cast<const uint16_t *>(z2),
                static_cast<uint16_t *>(out), tokens, hidden, inter, experts, topk, group,
                static_cast<int>(act), ids_out, w_out, workspace};
  a.sel_logits = sel_logits;
  a.finished = finished;
  a.b1 = static_cast<const uint16_t *>(b1);
  a.b2 = static_cast<const uint16_t *>(b2);
  a.renorm = norm == QG_MOE_RENORMALIZE ? 1 : 0;
  if (noalloc) return hip_status(qg::launch_moe_noalloc(a, as_stream(stream)));
  return hip_status(qg::launch_moe(a, as_stream(stream)));
}

qg_status qmoe_grouped(const void *x, const float *logits, const uint8_t *w1, const void *s1,
                       const void *z1, const uint8_t *w2, const void *s2, const void *z2,
                       void *out, int tokens, int hidden, int inter, int experts, int topk,
                       int group, qg_dtype act, int32_t *ids_out, float *w_out, void *workspace,
                       size_t ws_bytes, void *stream) {
  return moe_call(x, logits, nullptr, nullptr, w1, s1, z1, nullptr, w2, s2, z2, nullptr, out,
                  tokens, hidden, inter, experts, topk, group, QG_MOE_RENORMALIZE, act, ids_out,
                  w_out, workspace, ws_bytes, stream);
}

qg_status qmoe_grouped_noalloc(const void *x, const float *logits, const uint8_t *w1,
                               const void *s1, const void *z1, const uint8_t *w2, const void *s2,
                               const void *z2, void *out, int tokens, int hidden, int inter,
                               int experts, int topk, int group, qg_dtype act, int32_t *ids_out,
                               float *w_out, void *stream) {
  return moe_call(x, logits, nullptr, nullptr, w1, s1, z1, nullptr, w2, s2, z2, nullptr, out,
                  tokens, hidden, inter, experts, topk, group, QG_MOE_RENORMALIZE, act, ids_out,
                  w_out, nullptr, 0, stream, true);
}

qg_status qmoe_grouped_ex(const void *x, const float *logits, const float *sel_logits,
                          const uint8_t *finished, const uint8_t *w1, const void *s1,
                          const void *z1, const void *b1, const uint8_t *w2, const void *s2,
                          const void *z2, const void *b2, void *out, int tokens, int hidden,
                          int inter, int experts, int topk, int group, int norm, qg_dtype act,
                          int32_t *ids_out, float *w_out, void *workspace, size_t ws_bytes,
                          void *stream) {
  return moe_call(x, logits, sel_logits, finished, w1, s1, z1, b1, w2, s2, z2, b2, out, tokens,
                  hidden, inter, experts, topk, group, norm, act, ids_out, w_out, workspace,
                  ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Measurement probe
// ---------------------------------------------------------------------------
size_t qg_read_probe_blocks(size_t bytes) { return qg::read_probe_blocks(bytes); }

qg_status qg_read_probe(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  if (bytes % 16 != 0) return QG_ERR_SHAPE;
  if (!out || (bytes && !buf)) return QG_ERR_NULL;
  if ((buf && !aligned(buf, 16)) || !aligned(out, 4)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_read_probe(buf, bytes, out, as_stream(stream)));
}

qg_status qg_lds_probe(int waves, int iters, int blocks, unsigned long long *cycles, void *stream) {
  if (blocks < 1 || blocks > 65536 || iters < 8 || iters > (1 << 20) || iters % 8 != 0) return QG_ERR_SHAPE;
  if (waves != 4 && waves != 8 && waves != 16) return QG_ERR_MODE;
  if (!cycles) return QG_ERR_NULL;
  if (!aligned(cycles, 8)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_lds_probe(waves, iters, blocks, cycles, as_stream(stream)));
}

}  // extern "C"
