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
// eight values k0 + 8 * (lane / 16) + 0..7.  Rows >= M read row M - 1 (no
// divergent branch) and are zeroed.
__device__ __forceinline__ u32x4 load_afrag(const uint16_t *__restrict__ A, int M, int K, int m,
                                            int k) {
  const int row = m < M ? m : M - 1;
  const u32x4 v = *reinterpret_cast<const u32x4 *>(A + static_cast<size_t>(row) * K + k);
  const uint32_t keep = m < M ? 0xFFFFFFFFu : 0u;
  return u32x4{v.x & keep, v.y & keep, v.z & keep, v.w & keep};
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

// A chunk's NG consecutive 16-bit scale (or zero) values of one row, kept as
// packed words until use: one vector load when the row offset is aligned to
// it, else one load per value.
template <int NG>
struct Groups {
  static constexpr int W = (NG + 1) / 2;
  uint32_t w[W];
};

template <int NG, bool VEC>
__device__ __forceinline__ Groups<NG> load_groups(const uint16_t *__restrict__ p) {
  Groups<NG> g;
  if constexpr (VEC && NG == 8) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
    g.w[0] = v.x; g.w[1] = v.y; g.w[2] = v.z; g.w[3] = v.w;
  } else if constexpr (VEC && NG == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
    g.w[0] = v.x; g.w[1] = v.y;
  } else if constexpr (VEC && NG == 2) {
    g.w[0] = *reinterpret_cast<const uint32_t *>(p);
  } else {
#pragma unroll
    for (int i = 0; i < Groups<NG>::W; ++i) {
      const uint32_t lo = p[2 * i];
      const uint32_t hi = (2 * i + 1 < NG) ? p[2 * i + 1] : 0u;
      g.w[i] = lo | (hi << 16);
    }
  }
  return g;
}

// One 16-bit value in every group slot.
template <int NG>
__device__ __forceinline__ Groups<NG> splat_groups(uint16_t v) {
  Groups<NG> g;
  const uint32_t w = static_cast<uint32_t>(v) | (static_cast<uint32_t>(v) << 16);
#pragma unroll
  for (int i = 0; i < Groups<NG>::W; ++i) g.w[i] = w;
  return g;
}

template <int ACT, int NG>
__device__ __forceinline__ float group_value(const Groups<NG> &g, int i) {
  const uint32_t w = g.w[i >> 1];
  return bits_to_f32<ACT>(static_cast<uint16_t>((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

}  // namespace

// Launch bounds follow the plan: BPW 1 runs up to 16 waves, BPW 2 up to 8,
// BPW 4 up to 4, so the register budget grows with the chunk size (the int8
// kernel with one tile per workgroup runs up to 16 waves at any BPW).
template <int BPW>
constexpr int decode_threads() { return BPW == 1 ? 1024 : (BPW == 2 ? 512 : 256); }

// SPECIAL: the scale forms other than groupwise-with-zeros, decided at run
// time -- one scale (and zero) per channel when group != G (group = K, run
// with G = 128: every 128-k block then reads the channel's values), and no
// zeros when Z is null (w = (q - 8) s).  The common form compiles without
// these branches.
template <int ACT, int G, int BPW, int NT, bool VEC, bool SPECIAL>
__global__ __launch_bounds__(decode_threads<BPW>()) void k_decode_w4(const uint16_t *__restrict__ A,
                                                   const u32x4 *__restrict__ Bt,
                                                   const uint16_t *__restrict__ S,
                                                   const uint16_t *__restrict__ Z,
                                                   const uint16_t *__restrict__ bias, int bias_dt,
                                                   uint16_t *__restrict__ C, int M, int N, int K,
                                                   int group) {
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
    // Issue every weight and scale load of the NT tiles before any math, so
    // the workgroup pays one memory round trip per chunk, not one per tile.
    u32x4 bw[NT][BPW];
    Groups<NG> sv[NT], zv[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int nt = nt0 + i;
#pragma unroll
      for (int b = 0; b < BPW; ++b)
        bw[i][b] = __builtin_nontemporal_load(&Bt[(static_cast<size_t>(nt) * nb + kb0 + b) * 64 + lane]);
      const size_t srow = static_cast<size_t>(nt * 16 + nl) * ngroups + kb0 * GPB;
      if constexpr (SPECIAL) {
        if (group != G) {
          sv[i] = splat_groups<NG>(S[nt * 16 + nl]);
          zv[i] = Z ? splat_groups<NG>(Z[nt * 16 + nl]) : Groups<NG>{};
        } else {
          sv[i] = load_groups<NG, VEC>(S + srow);
          zv[i] = Z ? load_groups<NG, VEC>(Z + srow) : Groups<NG>{};
        }
      } else {
        sv[i] = load_groups<NG, VEC>(S + srow);
        zv[i] = load_groups<NG, VEC>(Z + srow);
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int b = 0; b < BPW; ++b)
#pragma unroll
        for (int h = 0; h < GPB; ++h) {
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int tt = 0; tt < TPG; ++tt) {
            const int t = h * TPG + tt;
            d = mfma16x16x32<ACT>(af[b][t], w4_word_to_operand<ACT>(bw[i][b][t]), d);
          }
          const int g = b * GPB + h;
          const float s = group_value<ACT, NG>(sv[i], g);
          const float zc = group_value<ACT, NG>(zv[i], g) - kOff * s;
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

// GS: 0 = one scale per channel, applied to the finished sum; 64 or 128 =
// one scale per (channel, K-group), applied to each 64-k block's partial
// product (the lane's channel is its output column, so the scale is a
// per-lane value).  EARLY (up to 4 rows): every load of a chunk is issued
// before its first wait.
template <int ACT, int BPW, int NT, int GS, bool EARLY>
__global__ __launch_bounds__(NT == 1 ? 1024 : decode_threads<BPW>()) void k_decode_w8(const uint16_t *__restrict__ A,
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
    u32x4 bw[NT][BPW];
    [[maybe_unused]] uint16_t sb[NT][BPW];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        bw[i][b] = __builtin_nontemporal_load(&Bt[(static_cast<size_t>(nt0 + i) * nb + kb0 + b) * 64 + lane]);
        if constexpr (GS > 0)
          sb[i][b] = S[static_cast<size_t>((nt0 + i) * 16 + nl) * (K / GS) + (kb0 + b) * 64 / GS];
      }
    // With EARLY all of the chunk's loads go out before its first wait; the
    // scheduler would otherwise split them over two or three round trips.
    // Measured on MI355X at K = 3584, N = 18944: M = 1 13.9 -> 13.4 us per
    // channel, 15.2 -> 14.4 us with group 128; at M = 16 with group 128 it
    // cost 4.6 % (20.8 -> 21.7 us), so the many-row forms keep the
    // scheduler's order.
    if constexpr (EARLY) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        if constexpr (GS == 0) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            u32x4 op = (ACT == kFP16) ? w8_run_to_f16(bw[i][b][2 * t], bw[i][b][2 * t + 1])
                                      : w8_run_to_bf16(bw[i][b][2 * t], bw[i][b][2 * t + 1]);
            acc[i] = mfma16x16x32<ACT>(af[b][t], op, acc[i]);
          }
        } else {
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            u32x4 op = (ACT == kFP16) ? w8_run_to_f16(bw[i][b][2 * t], bw[i][b][2 * t + 1])
                                      : w8_run_to_bf16(bw[i][b][2 * t], bw[i][b][2 * t + 1]);
            d = mfma16x16x32<ACT>(af[b][t], op, d);
          }
          const float sc = bits_to_f32<ACT>(sb[i][b]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][r] += sc * d[r];
        }
      }
  }
  constexpr int PER = NT * 256;
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * PER + i * 256 + r * 64 + lane] = acc[i][r];
  __syncthreads();
  reduce_store<ACT, NT>(red, nwaves, bias, bias_dt, GS > 0 ? nullptr : S, C, M, N, nt0);
}

// ---------------------------------------------------------------------------
// Streaming variant for many channel tiles (large N).  Each wave owns whole
// tiles of 16 channels over all of K, and consecutive waves of the grid take
// consecutive tiles, so at any moment the running waves sweep one contiguous
// window of the tiled weights -- the access pattern that streams best from
// HBM.  The activations (rows < M) and their per-group sums S_g live in LDS,
// written once per workgroup; no cross-wave reduction is needed.  K is walked
// in segments of SEG 128-k blocks whose codes are loaded together.
// ---------------------------------------------------------------------------
// R: accumulator rows per lane that can hold a live output (lane rows are
// m = 4 * (lane / 16) + r): M = 1 needs r = 0 only, M = 2 r < 2.  Only the
// live rows get the per-group scale update, which is most of the VALU work.
// Register budget for five resident waves per SIMD (five workgroups per CU):
// measured on MI355X at M = 1, N = 131072, K = 2048, 27.2-27.5 us against
// 27.5-27.6 with four and 27.9-28.3 with the compiler's default budget (three
// waves); six (28.9) and eight (31.6, with spills) were slower.  The first
// item's loads are issued before the activation staging, whose group sums
// are computed by all threads (a serial 64-value loop per group had every
// workgroup wait about 4k cycles before its first weight load): 2.5 % faster
// at M = 1, N = 131072 (27.6 against 28.3 us, same box); loading the next
// item before the current item's math (two items live) measured 5 % slower.
template <int ACT, int G, int SEG, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void k_decode_w4_stream(const uint16_t *__restrict__ A,
                                                          const u32x4 *__restrict__ Bt,
                                                          const uint16_t *__restrict__ S,
                                                          const uint16_t *__restrict__ Z,
                                                          const uint16_t *__restrict__ bias,
                                                          int bias_dt, uint16_t *__restrict__ C,
                                                          int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int GPB = 128 / G;           // groups per block
  constexpr int TPG = 4 / GPB;           // MFMA steps per group
  constexpr int NGS = SEG * GPB;         // groups per segment
  constexpr float kOff = w4_operand_offset<ACT>() + 8.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, j = lane >> 4;
  const int nb = K >> 7, ngroups = K / G, ntiles = N >> 4;
  const int arow = 2 * K + 16;           // padded LDS row (bytes)
  const int Mr = M < 16 ? M : 16;
  // LDS: rows 0 .. Mr - 1 of A, then a row of zeros (read by the lanes of
  // the padding rows m >= M, so every fragment read is unconditional), then
  // the group sums.
  float *sS = reinterpret_cast<float *>(lds + (Mr + 1) * arow);   // [ngroups][16]

  const int total_waves = gridDim.x * (blockDim.x >> 6);
  const int nseg = nb / SEG;
  static_assert(R == 1 || R == 2, "streaming decode serves M <= 2");

  // Codes and scales of one (tile, segment) item; all of an item's loads are
  // issued together, then consumed.
  struct Item {
    u32x4 bw[SEG];
    uint32_t sw[(NGS + 1) / 2], zw[(NGS + 1) / 2];
  };
  auto fetch = [&](int tile, int seg, Item &it) {
    const int kb0 = seg * SEG;
#pragma unroll
    for (int b = 0; b < SEG; ++b)
      it.bw[b] = __builtin_nontemporal_load(&Bt[(static_cast<size_t>(tile) * nb + kb0 + b) * 64 + lane]);
    const size_t off = static_cast<size_t>(tile * 16 + nl) * ngroups + kb0 * GPB;
    if constexpr (NGS >= 8) {
#pragma unroll
      for (int q = 0; q < NGS / 8; ++q) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(S + off + 8 * q);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(Z + off + 8 * q);
        it.sw[4 * q] = a.x; it.sw[4 * q + 1] = a.y; it.sw[4 * q + 2] = a.z; it.sw[4 * q + 3] = a.w;
        it.zw[4 * q] = b.x; it.zw[4 * q + 1] = b.y; it.zw[4 * q + 2] = b.z; it.zw[4 * q + 3] = b.w;
      }
    } else if constexpr (NGS == 4) {
      const u32x2 a = *reinterpret_cast<const u32x2 *>(S + off);
      const u32x2 b = *reinterpret_cast<const u32x2 *>(Z + off);
      it.sw[0] = a.x; it.sw[1] = a.y; it.zw[0] = b.x; it.zw[1] = b.y;
    } else {
      it.sw[0] = *reinterpret_cast<const uint32_t *>(S + off);
      it.zw[0] = *reinterpret_cast<const uint32_t *>(Z + off);
    }
  };

  // The first item's loads go out before the activations are staged, so
  // every wave has weights in flight from its first instructions on.
  int tile = blockIdx.x * (blockDim.x >> 6) + wave;
  Item cur;
  if (tile < ntiles) fetch(tile, 0, cur);

  // Activation rows -> LDS (16-byte chunks); S[g][m] = sum of group g of row
  // m, summed from the same chunks: each thread adds its 8 values and the
  // G / 8 consecutive lanes of a group combine by shuffles (a group never
  // straddles rows, and every pass runs on all threads, so the lanes a
  // shuffle reads are always active).  Rows m >= M read as zeros.
  constexpr int LPG = G / 8;             // lanes per group
  for (int e = threadIdx.x; e < ngroups * 16; e += blockDim.x)
    if ((e & 15) >= Mr) sS[e] = 0.f;
  for (int c = threadIdx.x; c < (K >> 3); c += blockDim.x)
    *reinterpret_cast<u32x4 *>(lds + Mr * arow + c * 16) = u32x4{0u, 0u, 0u, 0u};
  for (int base = 0; base < Mr * (K >> 3); base += blockDim.x) {
    const int c = base + static_cast<int>(threadIdx.x);
    const bool ok = c < Mr * (K >> 3);
    const int m = ok ? c / (K >> 3) : 0, k8 = ok ? c % (K >> 3) : 0;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) {
      v = *reinterpret_cast<const u32x4 *>(A + static_cast<size_t>(m) * K + k8 * 8);
      *reinterpret_cast<u32x4 *>(lds + m * arow + k8 * 16) = v;
    }
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      part += bits_to_f32<ACT>(static_cast<uint16_t>(v[q] & 0xFFFFu));
      part += bits_to_f32<ACT>(static_cast<uint16_t>(v[q] >> 16));
    }
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) part += __shfl_xor(part, off);
    if (ok && (k8 % LPG) == 0) sS[(k8 / LPG) * 16 + m] = part;
  }
  __syncthreads();

  const char *arow_p = lds + (nl < Mr ? nl : Mr) * arow + 16 * j;   // padding rows: the zero row
  const W4Consts wc = w4_consts<ACT>();

  // One item is live at a time: after an item's math, the loads of the next
  // one (the next segment of this tile, else the first of the wave's next
  // tile) are issued.
  for (; tile < ntiles; tile += total_waves) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int seg = 0; seg < nseg; ++seg) {
      const int kb0 = seg * SEG;
#pragma unroll
      for (int b = 0; b < SEG; ++b)
#pragma unroll
        for (int h = 0; h < GPB; ++h) {
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int tt = 0; tt < TPG; ++tt) {
            const int t = h * TPG + tt;
            const int k = (kb0 + b) * 128 + 32 * t;          // + 8 j via arow_p
            const u32x4 af = *reinterpret_cast<const u32x4 *>(arow_p + 2 * k);
            d = mfma16x16x32<ACT>(af, w4_word_to_operand<ACT>(cur.bw[b][t], wc), d);
          }
          const int gl = b * GPB + h, g = kb0 * GPB + gl;
          const uint32_t swd = cur.sw[gl >> 1], zwd = cur.zw[gl >> 1];
          const float sc = bits_to_f32<ACT>(static_cast<uint16_t>((gl & 1) ? (swd >> 16) : (swd & 0xFFFFu)));
          const float zc = bits_to_f32<ACT>(static_cast<uint16_t>((gl & 1) ? (zwd >> 16) : (zwd & 0xFFFFu))) - kOff * sc;
          if constexpr (R == 1) {
            acc[0] += sc * d[0] + zc * sS[g * 16 + 4 * j];
          } else {
            const f32x2 sg = *reinterpret_cast<const f32x2 *>(sS + g * 16 + 4 * j);
            acc[0] += sc * d[0] + zc * sg[0];
            acc[1] += sc * d[1] + zc * sg[1];
          }
        }
      if (seg + 1 < nseg) fetch(tile, seg + 1, cur);
      else if (tile + total_waves < ntiles) fetch(tile + total_waves, 0, cur);
    }
    const int n = tile * 16 + nl;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int m = 4 * j + r;
      if (m < M) {
        float v = acc[r];
        if (bias) v += bits_to_f32_dyn(bias[n], bias_dt);
        C[static_cast<size_t>(m) * N + n] = f32_to_bits<ACT>(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host dispatch.
// ---------------------------------------------------------------------------
namespace {

struct DecodePlan {
  int bpw, waves, nt;
};

// K is cut into chunks of `bpw` blocks shared out over `waves` waves; each
// workgroup owns `nt` tiles of 16 channels.  Measured on MI355X at K = 2048:
// two blocks per chunk (eight waves) beats one or four at every N, and two
// tiles per workgroup pays off once there are a few hundred tiles.
DecodePlan plan_decode(int nb, int ntiles) {
  DecodePlan p{1, 1, 1};
  p.bpw = nb % 2 == 0 ? 2 : 1;
  const int nchunks = nb / p.bpw;
  const int max_waves = 16 / p.bpw;
  p.waves = nchunks < max_waves ? nchunks : max_waves;
  p.nt = (ntiles >= 512 && ntiles % 2 == 0) ? 2 : 1;
  return p;
}

template <int ACT, int G, int R>
hipError_t launch_stream(const GemmArgs &a, hipStream_t s) {
  constexpr int SEG = 4;
  const int ntiles = a.N >> 4;
  const size_t lds = static_cast<size_t>(a.M + 1) * (2 * a.K + 16) + static_cast<size_t>(a.K / G) * 64;
  auto kern = k_decode_w4_stream<ACT, G, SEG, R>;
  // One resident pass: 5 workgroups of 4 waves per CU on 256 CUs.
  int grid = (ntiles + 3) / 4;
  if (grid > 1280) grid = 1280;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, a.A, static_cast<const u32x4 *>(a.B),
                     a.S, a.Z, a.bias, a.bias_dt, a.C, a.M, a.N, a.K);
  return hipGetLastError();
}

template <int ACT, int G>
hipError_t launch_stream_m(const GemmArgs &a, hipStream_t s) {
  return a.M == 1 ? launch_stream<ACT, G, 1>(a, s) : launch_stream<ACT, G, 2>(a, s);
}

}  // namespace

hipError_t launch_decode_w4(const GemmArgs &a, hipStream_t s) {
  const int nb = a.K >> 7, ntiles = a.N >> 4;
  // Per-channel scales (group = K) or no zeros: the run-time forms of the
  // split-K kernel (group 128 for per-channel).
  const bool special = a.Z == nullptr || (a.group != 64 && a.group != 128);
  // Streaming kernel: one or two rows, many tiles, K a multiple of 512,
  // scale rows 16-byte aligned, activations that fit in LDS.
  const bool aligned16 = !special &&
      ((reinterpret_cast<uintptr_t>(a.S) | reinterpret_cast<uintptr_t>(a.Z)) & 15) == 0 &&
      ((a.K / a.group) % 8) == 0;
  const bool fits = static_cast<size_t>(a.M + 1) * (2 * static_cast<size_t>(a.K) + 16) +
                        static_cast<size_t>(a.K / a.group) * 64 <= 64 * 1024;
  if (a.M <= 2 && ntiles >= 4096 && aligned16 && fits && nb % 4 == 0) {
    if (a.act == kBF16)
      return a.group == 64 ? launch_stream_m<kBF16, 64>(a, s) : launch_stream_m<kBF16, 128>(a, s);
    return a.group == 64 ? launch_stream_m<kFP16, 64>(a, s) : launch_stream_m<kFP16, 128>(a, s);
  }
  DecodePlan p = plan_decode(nb, ntiles);
  dim3 grid(ntiles / p.nt), block(64 * p.waves);
  size_t lds = static_cast<size_t>(p.waves) * p.nt * 256 * sizeof(float);
  const u32x4 *B = static_cast<const u32x4 *>(a.B);
  // Vector scale loads need the scale/zero bases aligned to a chunk's worth
  // of groups (the row offsets are multiples of it by construction).
  const int ng = p.bpw * (a.group == 64 ? 2 : 1);
  const uintptr_t amask = static_cast<uintptr_t>(2 * ng - 1);
  const bool vec = ((reinterpret_cast<uintptr_t>(a.S) | reinterpret_cast<uintptr_t>(a.Z)) & amask) == 0;
#define QG_DEC4(ACT_, G_, BPW_, NT_)                                                                 \
  do {                                                                                               \
    if (special)                                                                                     \
      hipLaunchKernelGGL((k_decode_w4<ACT_, G_, BPW_, NT_, false, true>), grid, block, lds, s, a.A,  \
                         B, a.S, a.Z, a.bias, a.bias_dt, a.C, a.M, a.N, a.K, a.group);              \
    else if (vec)                                                                                    \
      hipLaunchKernelGGL((k_decode_w4<ACT_, G_, BPW_, NT_, true, false>), grid, block, lds, s, a.A,  \
                         B, a.S, a.Z, a.bias, a.bias_dt, a.C, a.M, a.N, a.K, a.group);              \
    else                                                                                             \
      hipLaunchKernelGGL((k_decode_w4<ACT_, G_, BPW_, NT_, false, false>), grid, block, lds, s, a.A, \
                         B, a.S, a.Z, a.bias, a.bias_dt, a.C, a.M, a.N, a.K, a.group);              \
  } while (0)
#define QG_DEC4_NT(ACT_, G_, BPW_)                   \
  if (p.nt == 2) QG_DEC4(ACT_, G_, BPW_, 2);         \
  else QG_DEC4(ACT_, G_, BPW_, 1);
#define QG_DEC4_BPW(ACT_, G_)                        \
  if (p.bpw == 2) { QG_DEC4_NT(ACT_, G_, 2) }        \
  else { QG_DEC4_NT(ACT_, G_, 1) }
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
  DecodePlan p = plan_decode(nb, ntiles);
  // One tile per workgroup (a few hundred tiles or fewer) and up to 4 rows:
  // up to 16 waves share K, so each wave runs half as many chunks, each one
  // a memory round trip.  Measured on MI355X at K = 3584, N = 3584: M = 1
  // 5.38 -> 4.80 us (group 128: 5.41 -> 5.04), M = 4 5.46 -> 4.98; at M = 16
  // and with two tiles per workgroup (N = 18944) no gain or a loss.
  if (p.nt == 1 && a.M <= 4) {
    const int nch = nb / p.bpw;
    p.waves = nch < 16 ? nch : 16;
  }
  dim3 grid(ntiles / p.nt), block(64 * p.waves);
  size_t lds = static_cast<size_t>(p.waves) * p.nt * 256 * sizeof(float);
  const u32x4 *B = static_cast<const u32x4 *>(a.B);
#define QG_DEC8G(ACT_, BPW_, NT_, GS_)                                                                  \
  do {                                                                                                  \
    if (a.M <= 4)                                                                                       \
      hipLaunchKernelGGL((k_decode_w8<ACT_, BPW_, NT_, GS_, true>), grid, block, lds, s, a.A, B, a.S,  \
                         a.bias, a.bias_dt, a.C, a.M, a.N, a.K);                                       \
    else                                                                                                \
      hipLaunchKernelGGL((k_decode_w8<ACT_, BPW_, NT_, GS_, false>), grid, block, lds, s, a.A, B, a.S, \
                         a.bias, a.bias_dt, a.C, a.M, a.N, a.K);                                       \
  } while (0)
#define QG_DEC8(ACT_, BPW_, NT_)                                \
  do {                                                          \
    if (a.group == 64) QG_DEC8G(ACT_, BPW_, NT_, 64);           \
    else if (a.group == 128) QG_DEC8G(ACT_, BPW_, NT_, 128);    \
    else QG_DEC8G(ACT_, BPW_, NT_, 0);                          \
  } while (0)
#define QG_DEC8_NT(ACT_, BPW_)                       \
  if (p.nt == 2) QG_DEC8(ACT_, BPW_, 2);             \
  else QG_DEC8(ACT_, BPW_, 1);
#define QG_DEC8_BPW(ACT_)                            \
  if (p.bpw == 2) { QG_DEC8_NT(ACT_, 2) }            \
  else { QG_DEC8_NT(ACT_, 1) }
  if (a.act == kBF16) { QG_DEC8_BPW(kBF16); } else { QG_DEC8_BPW(kFP16); }
#undef QG_DEC8_BPW
#undef QG_DEC8_NT
#undef QG_DEC8
#undef QG_DEC8G
  return hipGetLastError();
}

}  // namespace qg
