// decode.hip -- small-M (M <= 16) weight-only quantized GEMM for gfx950.
//
// Decode reads every weight once per token, so its speed is set by how fast
// the packed weights stream from HBM (vllm-omni cpu_int4.py, module
// docstring: single-stream decode is a bandwidth problem; "acext User Guide
// (v1.7)" 1.3.1: fewer weight bytes help memory-bound cases).  The kernels
// here therefore never materialise a dequantized weight.  Each 32-bit word of
// tiled int4 codes becomes eight exact matrix-core operands (offset + q) with
// one AND-OR per pair, and the affine dequant w = (q - 8) * s + z is applied
// per K-group to the fp32 partial sums instead:
//
//   sum_{k in g} a_k * w_k = s * D_g + (z - (off + 8) * s) * S_g,
//   D_g = sum_{k in g} a_k * (off + q_k),   S_g = sum_{k in g} a_k,
//
// where D_g comes from v_mfma_f32_16x16x32 on the converted codes and S_g
// from the same instruction against a column of ones.  int8 per-channel codes
// become exact fp16 q (byte permute + one packed subtract), and the single
// per-channel scale multiplies the finished sum.
//
// Work split: a workgroup owns NT tiles of 16 output channels.  K is cut into
// chunks of BPW blocks dealt out round-robin to the workgroup's waves; each
// wave loads a chunk's activation fragments and S_g once and applies them to
// all NT tiles; the per-wave partial sums are added through LDS at the end.
#include "qg_common.hpp"
#include "qg_launch.hpp"

namespace qg {

namespace {

// Activation fragment of v_mfma_f32_16x16x32: row m = lane % 16 holds the
// eight values k0 + 8 * (lane / 16) + 0..7.  Rows >= M are zero.
__device__ __forceinline__ u32x4 load_afrag(const uint16_t *__restrict__ A, int M, int K, int m,
                                            int k) {
  if (m < M) return *reinterpret_cast<const u32x4 *>(A + static_cast<size_t>(m) * K + k);
  return u32x4{0u, 0u, 0u, 0u};
}

// Sum the per-wave partials in LDS, add bias, round, store rows < M.
// red layout: [wave][tile][r][lane] floats.
template <int ACT, int NT>
__device__ __forceinline__ void reduce_store(float *red, int nwaves, const uint16_t *bias,
                                             int bias_dt, const uint16_t *colscale, uint16_t *C,
                                             int M, int N, int nt0) {
  constexpr int PER = NT * 256;
  for (int e = threadIdx.x; e < PER; e += blockDim.x) {
    int i = e >> 8, r = (e >> 6) & 3, lane = e & 63;
    int m = 4 * (lane >> 4) + r;
    if (m >= M) continue;
    float v = 0.f;
    for (int w = 0; w < nwaves; ++w) v += red[w * PER + e];
    int n = (nt0 + i) * 16 + (lane & 15);
    if (colscale) v *= bits_to_f32<ACT>(colscale[n]);
    if (bias) v += bits_to_f32_dyn(bias[n], bias_dt);
    C[static_cast<size_t>(m) * N + n] = f32_to_bits<ACT>(v);
  }
}

}  // namespace

template <int ACT, int G, int BPW, int NT>
__global__ __launch_bounds__(512) void k_decode_w4(const uint16_t *__restrict__ A,
                                                   const u32x4 *__restrict__ Bt,
                                                   const uint16_t *__restrict__ S,
                                                   const uint16_t *__restrict__ Z,
                                                   const uint16_t *__restrict__ bias, int bias_dt,
                                                   uint16_t *__restrict__ C, int M, int N, int K) {
  extern __shared__ float red[];
  constexpr int GPB = 128 / G;        // groups per 128-k block
  constexpr int TPG = 4 / GPB;        // 32-k MFMA steps per group
  constexpr int NG = BPW * GPB;       // groups per chunk
  constexpr float kOff = w4_operand_offset<ACT>() + 8.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int nl = lane & 15, j = lane >> 4;
  const int nb = K >> 7, ngroups = K / G, nchunks = nb / BPW;
  const int nt0 = blockIdx.x * NT;
  const u32x4 ones = {one_pair<ACT>(), one_pair<ACT>(), one_pair<ACT>(), one_pair<ACT>()};

  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int chunk = wave; chunk < nchunks; chunk += nwaves) {
    const int kb0 = chunk * BPW;
    // Activation fragments and per-group activation sums for this K chunk,
    // shared by the NT channel tiles below.
    u32x4 af[BPW][4];
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
      for (int t = 0; t < 4; ++t) af[b][t] = load_afrag(A, M, K, nl, (kb0 + b) * 128 + 32 * t + 8 * j);
    f32x4 sg[NG];
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
      for (int h = 0; h < GPB; ++h) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) d = mfma16x16x32<ACT>(af[b][h * TPG + tt], ones, d);
        sg[b * GPB + h] = d;
      }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int nt = nt0 + i;
      u32x4 bw[BPW];
#pragma unroll
      for (int b = 0; b < BPW; ++b) bw[b] = Bt[(static_cast<size_t>(nt) * nb + kb0 + b) * 64 + lane];
      const size_t srow = static_cast<size_t>(nt * 16 + nl) * ngroups + kb0 * GPB;
      float sv[NG], zv[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        sv[g] = bits_to_f32<ACT>(S[srow + g]);
        zv[g] = bits_to_f32<ACT>(Z[srow + g]);
      }
#pragma unroll
      for (int b = 0; b < BPW; ++b)
#pragma unroll
        for (int h = 0; h < GPB; ++h) {
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int tt = 0; tt < TPG; ++tt) {
            const int t = h * TPG + tt;
            d = mfma16x16x32<ACT>(af[b][t], w4_word_to_operand<ACT>(bw[b][t]), d);
          }
          const int g = b * GPB + h;
          const float s = sv[g];
          const float zc = zv[g] - kOff * s;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][r] += s * d[r] + zc * sg[g][r];
        }
    }
  }
  constexpr int PER = NT * 256;
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * PER + i * 256 + r * 64 + lane] = acc[i][r];
  __syncthreads();
  reduce_store<ACT, NT>(red, nwaves, bias, bias_dt, nullptr, C, M, N, nt0);
}

template <int ACT, int BPW, int NT>
__global__ __launch_bounds__(512) void k_decode_w8(const uint16_t *__restrict__ A,
                                                   const u32x4 *__restrict__ Bt,
                                                   const uint16_t *__restrict__ S,
                                                   const uint16_t *__restrict__ bias, int bias_dt,
                                                   uint16_t *__restrict__ C, int M, int N, int K) {
  extern __shared__ float red[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int nl = lane & 15, j = lane >> 4;
  const int nb = K >> 6, nchunks = nb / BPW;
  const int nt0 = blockIdx.x * NT;

  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int chunk = wave; chunk < nchunks; chunk += nwaves) {
    const int kb0 = chunk * BPW;
    u32x4 af[BPW][2];
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
      for (int t = 0; t < 2; ++t) af[b][t] = load_afrag(A, M, K, nl, (kb0 + b) * 64 + 32 * t + 8 * j);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int nt = nt0 + i;
      u32x4 bw[BPW];
#pragma unroll
      for (int b = 0; b < BPW; ++b) bw[b] = Bt[(static_cast<size_t>(nt) * nb + kb0 + b) * 64 + lane];
#pragma unroll
      for (int b = 0; b < BPW; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 op = (ACT == kFP16) ? w8_run_to_f16(bw[b][2 * t], bw[b][2 * t + 1])
                                    : w8_run_to_bf16(bw[b][2 * t], bw[b][2 * t + 1]);
          acc[i] = mfma16x16x32<ACT>(af[b][t], op, acc[i]);
        }
    }
  }
  constexpr int PER = NT * 256;
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * PER + i * 256 + r * 64 + lane] = acc[i][r];
  __syncthreads();
  reduce_store<ACT, NT>(red, nwaves, bias, bias_dt, S, C, M, N, nt0);
}

// ---------------------------------------------------------------------------
// Host dispatch.
// ---------------------------------------------------------------------------
namespace {

struct DecodePlan {
  int bpw, waves, nt;
};

// K is cut into chunks of `bpw` blocks shared out over `waves` waves; each
// workgroup owns `nt` tiles of 16 channels.  Small N: thin chunks and many
// waves, so that every byte is requested at once; large N: fat chunks and
// several tiles per workgroup, so activation fragments are reused.
DecodePlan plan_decode(int nb, int ntiles, int max_bpw) {
  DecodePlan p{1, 1, 1};
  int bpw = ntiles >= 2048 ? 4 : (ntiles >= 512 ? 2 : 1);
  if (bpw > max_bpw) bpw = max_bpw;
  while (bpw > 1 && nb % bpw != 0) bpw >>= 1;
  p.bpw = bpw;
  const int nchunks = nb / bpw;
  p.waves = nchunks < 8 ? nchunks : 8;
  int nt = ntiles >= 4096 ? 4 : (ntiles >= 2048 ? 2 : 1);
  while (nt > 1 && ntiles % nt != 0) nt >>= 1;
  p.nt = nt;
  return p;
}

}  // namespace

hipError_t launch_decode_w4(const GemmArgs &a, hipStream_t s) {
  const int nb = a.K >> 7, ntiles = a.N >> 4;
  DecodePlan p = plan_decode(nb, ntiles, 4);
  dim3 grid(ntiles / p.nt), block(64 * p.waves);
  size_t lds = static_cast<size_t>(p.waves) * p.nt * 256 * sizeof(float);
  const u32x4 *B = static_cast<const u32x4 *>(a.B);
#define QG_DEC4(ACT_, G_, BPW_, NT_)                                                          \
  hipLaunchKernelGGL((k_decode_w4<ACT_, G_, BPW_, NT_>), grid, block, lds, s, a.A, B, a.S, a.Z, \
                     a.bias, a.bias_dt, a.C, a.M, a.N, a.K)
#define QG_DEC4_NT(ACT_, G_, BPW_)                   \
  switch (p.nt) {                                    \
    case 4: QG_DEC4(ACT_, G_, BPW_, 4); break;       \
    case 2: QG_DEC4(ACT_, G_, BPW_, 2); break;       \
    default: QG_DEC4(ACT_, G_, BPW_, 1); break;      \
  }
#define QG_DEC4_BPW(ACT_, G_)                        \
  switch (p.bpw) {                                   \
    case 4: QG_DEC4_NT(ACT_, G_, 4); break;          \
    case 2: QG_DEC4_NT(ACT_, G_, 2); break;          \
    default: QG_DEC4_NT(ACT_, G_, 1); break;         \
  }
  if (a.act == kBF16) {
    if (a.group == 64) { QG_DEC4_BPW(kBF16, 64); } else { QG_DEC4_BPW(kBF16, 128); }
  } else {
    if (a.group == 64) { QG_DEC4_BPW(kFP16, 64); } else { QG_DEC4_BPW(kFP16, 128); }
  }
#undef QG_DEC4_BPW
#undef QG_DEC4_NT
#undef QG_DEC4
  return hipGetLastError();
}

hipError_t launch_decode_w8(const GemmArgs &a, hipStream_t s) {
  const int nb = a.K >> 6, ntiles = a.N >> 4;
  DecodePlan p = plan_decode(nb, ntiles, 4);
  dim3 grid(ntiles / p.nt), block(64 * p.waves);
  size_t lds = static_cast<size_t>(p.waves) * p.nt * 256 * sizeof(float);
  const u32x4 *B = static_cast<const u32x4 *>(a.B);
#define QG_DEC8(ACT_, BPW_, NT_)                                                               \
  hipLaunchKernelGGL((k_decode_w8<ACT_, BPW_, NT_>), grid, block, lds, s, a.A, B, a.S, a.bias, \
                     a.bias_dt, a.C, a.M, a.N, a.K)
#define QG_DEC8_NT(ACT_, BPW_)                       \
  switch (p.nt) {                                    \
    case 4: QG_DEC8(ACT_, BPW_, 4); break;           \
    case 2: QG_DEC8(ACT_, BPW_, 2); break;           \
    default: QG_DEC8(ACT_, BPW_, 1); break;          \
  }
#define QG_DEC8_BPW(ACT_)                            \
  switch (p.bpw) {                                   \
    case 4: QG_DEC8_NT(ACT_, 4); break;              \
    case 2: QG_DEC8_NT(ACT_, 2); break;              \
    default: QG_DEC8_NT(ACT_, 1); break;             \
  }
  if (a.act == kBF16) { QG_DEC8_BPW(kBF16); } else { QG_DEC8_BPW(kFP16); }
#undef QG_DEC8_BPW
#undef QG_DEC8_NT
#undef QG_DEC8
  return hipGetLastError();
}

}  // namespace qg
