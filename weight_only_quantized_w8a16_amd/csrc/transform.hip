// transform.hip -- load-side repack into the tiled layouts of include/qgemm.h,
// its inverse, and the bit-exact dequantization hook.
//
// The repack is a pure permutation done once when weights are loaded, so that
// the GEMM kernels never shuffle nibbles per call (the motivation vllm-omni
// cpu_int4.py gives for its to_split_halves de-interleave).  The dequant rule
// is the one of that file's module docstring: w = (q - 8) * scale + zero, and
// for int8 "acext User Guide (v1.7)" 1.3.1: w = q * scale per channel.
#include "qg_common.hpp"
#include "qg_launch.hpp"

namespace qg {

// One thread per tiled 32-bit word.  Word index -> (block, lane slot, t).
__global__ void k_repack_w4(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst,
                            int n, int k, long long words) {
  long long w = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (w >= words) return;
  int kblocks = k >> 7;
  long long blk = w >> 8;
  int slot = static_cast<int>((w >> 2) & 63), t = static_cast<int>(w & 3);
  int nt = static_cast<int>(blk / kblocks), kb = static_cast<int>(blk % kblocks);
  int row = nt * 16 + (slot & 15), j = slot >> 4;
  int k0 = kb * 128 + 32 * t + 8 * j;                    // 8 codes = 1 source word
  uint32_t v = src[(static_cast<size_t>(row) * (k >> 1) + (k0 >> 1)) >> 2];
  dst[w] = w4_to_tiled_word(v);
}

__global__ void k_unrepack_w4(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst,
                              int n, int k, long long words) {
  long long w = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (w >= words) return;
  int kblocks = k >> 7;
  long long blk = w >> 8;
  int slot = static_cast<int>((w >> 2) & 63), t = static_cast<int>(w & 3);
  int nt = static_cast<int>(blk / kblocks), kb = static_cast<int>(blk % kblocks);
  int row = nt * 16 + (slot & 15), j = slot >> 4;
  int k0 = kb * 128 + 32 * t + 8 * j;
  dst[(static_cast<size_t>(row) * (k >> 1) + (k0 >> 1)) >> 2] = w4_from_tiled_word(src[w]);
}

// One thread per 8-byte run (block, slot, t): 8 consecutive k of one row.
__global__ void k_repack_w8(const uint2 *__restrict__ src, uint2 *__restrict__ dst, int n, int k,
                            long long runs, int flip_from_tiled) {
  long long r = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= runs) return;
  int kblocks = k >> 6;
  long long blk = r >> 7;
  int slot = static_cast<int>((r >> 1) & 63), t = static_cast<int>(r & 1);
  int nt = static_cast<int>(blk / kblocks), kb = static_cast<int>(blk % kblocks);
  int row = nt * 16 + (slot & 15), j = slot >> 4;
  int k0 = kb * 64 + 32 * t + 8 * j;
  size_t lin = (static_cast<size_t>(row) * k + k0) >> 3;
  if (!flip_from_tiled) {
    uint2 v = src[lin];
    v.x ^= 0x80808080u;
    v.y ^= 0x80808080u;
    dst[r] = v;
  } else {
    uint2 v = src[r];
    v.x ^= 0x80808080u;
    v.y ^= 0x80808080u;
    dst[lin] = v;
  }
}

// int8 weights stored K-major, [k, n] row-major (the orientation of the
// "acext User Guide (v1.7)" examples: 1.3.1 preprocesses a row-major {k, n}
// weight, and 2.1.2 allocates qweight as [input size, output size]) <-> the
// tiled layout of qrepack_w8.  A workgroup moves a 64 (k) x 64 (n) byte tile
// through LDS, so both sides are read and written in whole 16-byte pieces:
// the [k, n] rows as 16-byte chunks, the tiled side as the four 1 KiB blocks
// of the tile's 16-channel groups, 8-byte runs per thread.
template <bool TO_TILED>
__global__ __launch_bounds__(256) void k_repack_w8_kn(const uint8_t *__restrict__ src,
                                                      uint8_t *__restrict__ dst, int n, int k) {
  __shared__ uint32_t tile[64][17];          // [k in the tile][n in the tile], 68-byte rows
  uint8_t *tb = reinterpret_cast<uint8_t *>(&tile[0][0]);
  const int n0 = blockIdx.x * 64, kb = blockIdx.y, tid = threadIdx.x;
  const int kr = tid >> 2, c = tid & 3;      // [k, n] side: row kr, 16-byte chunk c
  const bool row_chunk = n0 + 16 * c < n;    // n % 16 == 0: chunks are whole or absent
  const size_t kn_off = static_cast<size_t>(kb * 64 + kr) * n + n0 + 16 * c;
  auto run_of = [&](int h, int &i, int &nl, int &kl, size_t &toff) {
    const int q = tid + 256 * h;             // run q of the tile's 512
    const int rr = q & 127, slot = rr >> 1, t = rr & 1;
    i = q >> 7;                               // 16-channel group within the tile
    nl = slot & 15;
    kl = 32 * t + 8 * (slot >> 4);
    toff = (static_cast<size_t>((n0 >> 4) + i) * (k >> 6) + kb) * 1024u + rr * 8;
  };
  if constexpr (TO_TILED) {
    if (row_chunk) {
      const uint4 v = *reinterpret_cast<const uint4 *>(src + kn_off);
      tile[kr][4 * c] = v.x; tile[kr][4 * c + 1] = v.y; tile[kr][4 * c + 2] = v.z; tile[kr][4 * c + 3] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int i, nl, kl;
      size_t toff;
      run_of(h, i, nl, kl, toff);
      if (n0 + 16 * i >= n) continue;
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e >> 2] |= static_cast<uint32_t>(tb[(kl + e) * 68 + 16 * i + nl] ^ 0x80u) << (8 * (e & 3));
      *reinterpret_cast<uint2 *>(dst + toff) = make_uint2(w[0], w[1]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int i, nl, kl;
      size_t toff;
      run_of(h, i, nl, kl, toff);
      if (n0 + 16 * i >= n) continue;
      const uint2 v = *reinterpret_cast<const uint2 *>(src + toff);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tb[(kl + e) * 68 + 16 * i + nl] = static_cast<uint8_t>(((e < 4 ? v.x : v.y) >> (8 * (e & 3))) ^ 0x80u);
    }
    __syncthreads();
    if (row_chunk)
      *reinterpret_cast<uint4 *>(dst + kn_off) =
          make_uint4(tile[kr][4 * c], tile[kr][4 * c + 1], tile[kr][4 * c + 2], tile[kr][4 * c + 3]);
  }
}

static inline unsigned grid_for(long long items, int block) {
  return static_cast<unsigned>((items + block - 1) / block);
}

hipError_t launch_repack_w8_kn(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s) {
  hipLaunchKernelGGL(k_repack_w8_kn<true>, dim3((n + 63) / 64, k / 64), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t *>(src), reinterpret_cast<uint8_t *>(dst), n, k);
  return hipGetLastError();
}
hipError_t launch_unrepack_w8_kn(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s) {
  hipLaunchKernelGGL(k_repack_w8_kn<false>, dim3((n + 63) / 64, k / 64), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t *>(src), reinterpret_cast<uint8_t *>(dst), n, k);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Groupwise min/max quantizer (vllm-omni cpu_int4.py, quantize_groupwise):
// per K-group, scale = max(hi - lo, 1e-9) / 15, zero = lo + 8 scale,
// q = round-half-even((w - lo) / scale) clamped to [0, 15], in fp32 (the
// codes are those of the correctly rounded division; see below).  A run is
// 8 consecutive values of a row -- one 32-bit word of the portable layout;
// GROUP / 8 consecutive lanes hold a group's runs and exchange their
// partial minimum and maximum.  Groups never straddle rows
// (k % GROUP == 0), so the flat run index r is also the word index and
// r / (GROUP / 8) the group index.
// ---------------------------------------------------------------------------
template <int WT>
__device__ __forceinline__ void load8(const void *W, long long r, float (&x)[8]) {
  if constexpr (WT == QG_FP32) {
    const float4 *p = static_cast<const float4 *>(W) + 2 * r;
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 v = static_cast<const uint4 *>(W)[r];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bits_to_f32<WT>(static_cast<uint16_t>(w[i] & 0xFFFFu));
      x[2 * i + 1] = bits_to_f32<WT>(static_cast<uint16_t>(w[i] >> 16));
    }
  }
}

template <int SZ>
__device__ __forceinline__ void store_sz(void *dst, long long i, float v) {
  if constexpr (SZ == QG_FP32) static_cast<float *>(dst)[i] = v;
  else static_cast<uint16_t *>(dst)[i] = f32_to_bits<SZ>(v);
}

template <int WT, int SZ, int GROUP>
__global__ __launch_bounds__(256) void k_quantize_w4(const void *__restrict__ W,
                                                     uint32_t *__restrict__ packed,
                                                     void *__restrict__ scale,
                                                     void *__restrict__ zero, long long runs) {
  constexpr int LPG = GROUP / 8;   // threads per group
  const long long r = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= runs) return;           // whole groups only: runs is a multiple of LPG
  float x[8];
  load8<WT>(W, r, x);
  // Group extremes.  The NaN-propagating minimum / maximum take the values
  // as they are (no quieting pass), and agree with < / > on the finite
  // inputs the quantizer is defined for.
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    lo = __builtin_elementwise_minimum(lo, x[e]);
    hi = __builtin_elementwise_maximum(hi, x[e]);
  }
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    lo = __builtin_elementwise_minimum(lo, __shfl_xor(lo, off));
    hi = __builtin_elementwise_maximum(hi, __shfl_xor(hi, off));
  }
  float range = hi - lo;
  if (range < 1e-9f) range = 1e-9f;
  const float s = range / 15.0f;   // correctly rounded: it is an output
  const float z = lo + 8.0f * s;
  // Each code is rint of the correctly rounded quotient d = fl((w - lo) / s).
  // Here 0 <= w - lo <= range (rounding is monotone) and s is range / 15
  // rounded, so d lies in [0, 15 (1 + 2^-23)].  Adding 1.5 * 2^23 rounds a
  // value of that range to an integer, ties to even, which then sits in the
  // low byte of the sum's bits.  With rcp the hardware reciprocal of s
  // (error below 1 ulp), the product (w - lo) * rcp is within 4e-6 of d and
  // is rounded by one fused multiply-add; unless it lies within 1e-5 of a
  // half-integer (its distance to the chosen integer, from a second fused
  // multiply-add, is then below 0.5 - 1e-5), it rounds to the same integer
  // as d.  Otherwise the run's quotients are recomputed by division (rare:
  // about one run in 6000).
  constexpr float kRound = 12582912.0f;   // 1.5 * 2^23
  const float rcp = __builtin_amdgcn_rcpf(s);
  float a[8], t[8];
  float worst = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = x[e] - lo;
    t[e] = __builtin_fmaf(a[e], rcp, kRound);
    worst = fmaxf(worst, fabsf(__builtin_fmaf(a[e], rcp, kRound - t[e])));
  }
  if (worst > 0.5f - 1e-5f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = a[e] / s + kRound;
  }
  // Low bytes hold the codes: pair them into nibbles, then gather the bytes.
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p[i] = (__float_as_uint(t[2 * i + 1]) << 4) | __float_as_uint(t[2 * i]);
  const uint32_t lo16 = __builtin_amdgcn_perm(p[1], p[0], 0x0C0C0400u);
  const uint32_t hi16 = __builtin_amdgcn_perm(p[3], p[2], 0x0C0C0400u);
  packed[r] = __builtin_amdgcn_perm(hi16, lo16, 0x05040100u);
  if ((r & (LPG - 1)) == 0) {
    store_sz<SZ>(scale, r / LPG, s);
    store_sz<SZ>(zero, r / LPG, z);
  }
}

hipError_t launch_quantize_w4(const void *W, uint8_t *packed, void *scale, void *zero, int n,
                              int k, int group, int w_dt, int sz_dt, hipStream_t s) {
  const long long runs = static_cast<long long>(n) * k / 8;
  dim3 g(grid_for(runs, 256)), b(256);
  uint32_t *P = reinterpret_cast<uint32_t *>(packed);
#define QG_Q4(WT_, SZ_)                                                                          \
  do {                                                                                           \
    if (group == 64)                                                                             \
      hipLaunchKernelGGL((k_quantize_w4<WT_, SZ_, 64>), g, b, 0, s, W, P, scale, zero, runs);  \
    else                                                                                         \
      hipLaunchKernelGGL((k_quantize_w4<WT_, SZ_, 128>), g, b, 0, s, W, P, scale, zero, runs); \
  } while (0)
#define QG_Q4_SZ(WT_)                                   \
  do {                                                  \
    if (sz_dt == QG_FP32) QG_Q4(WT_, QG_FP32);          \
    else if (sz_dt == QG_BF16) QG_Q4(WT_, QG_BF16);     \
    else QG_Q4(WT_, QG_FP16);                           \
  } while (0)
  if (w_dt == QG_FP32) QG_Q4_SZ(QG_FP32);
  else if (w_dt == QG_BF16) QG_Q4_SZ(QG_BF16);
  else QG_Q4_SZ(QG_FP16);
#undef QG_Q4_SZ
#undef QG_Q4
  return hipGetLastError();
}

hipError_t launch_repack_w4(const uint8_t *src, uint8_t *dst, int n, int k, hipStream_t s) {
  long long words = static_cast<long long>(n) * k / 8;
  hipLaunchKernelGGL(k_repack_w4, dim3(grid_for(words, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t *>(src), reinterpret_cast<uint32_t *>(dst),
                     n, k, words);
  return hipGetLastError();
}
hipError_t launch_unrepack_w4(const uint8_t *src, uint8_t *dst, int n, int k, hipStream_t s) {
  long long words = static_cast<long long>(n) * k / 8;
  hipLaunchKernelGGL(k_unrepack_w4, dim3(grid_for(words, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t *>(src), reinterpret_cast<uint32_t *>(dst),
                     n, k, words);
  return hipGetLastError();
}
hipError_t launch_repack_w8(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s) {
  long long runs = static_cast<long long>(n) * k / 8;
  hipLaunchKernelGGL(k_repack_w8, dim3(grid_for(runs, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint2 *>(src), reinterpret_cast<uint2 *>(dst), n, k,
                     runs, 0);
  return hipGetLastError();
}
hipError_t launch_unrepack_w8(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s) {
  long long runs = static_cast<long long>(n) * k / 8;
  hipLaunchKernelGGL(k_repack_w8, dim3(grid_for(runs, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint2 *>(src), reinterpret_cast<uint2 *>(dst), n, k,
                     runs, 1);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequant hook.  One thread per (row, 8 consecutive k).  fp32 value
// fmaf(q - 8, s, z): the product is exact in fp32, so the fused form rounds
// exactly once, like the plain definition.  16-bit outputs round to nearest
// even from that fp32 value.
// ---------------------------------------------------------------------------
template <int ACT, int OUT>
__global__ void k_dequant_w4(const uint8_t *__restrict__ B, const uint16_t *__restrict__ S,
                             const uint16_t *__restrict__ Z, void *__restrict__ W, int n, int k,
                             int group, long long runs) {
  long long r = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= runs) return;
  int per_row = k >> 3;
  int row = static_cast<int>(r / per_row), k0 = static_cast<int>(r % per_row) * 8;
  uint32_t word = *reinterpret_cast<const uint32_t *>(B + w4_word_offset(row, k0, k));
  size_t gi = static_cast<size_t>(row) * (k / group) + k0 / group;
  float s = bits_to_f32<ACT>(S[gi]);
  float z = Z ? bits_to_f32<ACT>(Z[gi]) : 0.0f;   // no zeros: scale-only
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    v[e] = __builtin_fmaf(static_cast<float>(static_cast<int>(w4_tiled_code(word, e)) - 8), s, z);
  size_t o = static_cast<size_t>(row) * k + k0;
  if constexpr (OUT == QG_FP32) {
    float4 *d = reinterpret_cast<float4 *>(static_cast<float *>(W) + o);
    d[0] = make_float4(v[0], v[1], v[2], v[3]);
    d[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 pk;
    pk.x = pack2<OUT>(v[0], v[1]);
    pk.y = pack2<OUT>(v[2], v[3]);
    pk.z = pack2<OUT>(v[4], v[5]);
    pk.w = pack2<OUT>(v[6], v[7]);
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(W) + o) = pk;
  }
}

// group 0: one scale per channel; else one per (channel, K-group).
template <int ACT, int OUT>
__global__ void k_dequant_w8(const int8_t *__restrict__ B, const uint16_t *__restrict__ S,
                             void *__restrict__ W, int n, int k, int group, long long runs) {
  long long r = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= runs) return;
  int per_row = k >> 3;
  int row = static_cast<int>(r / per_row), k0 = static_cast<int>(r % per_row) * 8;
  uint2 run = *reinterpret_cast<const uint2 *>(B + w8_run_offset(row, k0, k));
  float s = bits_to_f32<ACT>(group > 0 ? S[static_cast<size_t>(row) * (k / group) + k0 / group] : S[row]);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t word = e < 4 ? run.x : run.y;
    int q = static_cast<int>((word >> (8 * (e & 3))) & 0xFFu) - 128;
    v[e] = static_cast<float>(q) * s;   // exact: 8 x 11 significant bits
  }
  size_t o = static_cast<size_t>(row) * k + k0;
  if constexpr (OUT == QG_FP32) {
    float4 *d = reinterpret_cast<float4 *>(static_cast<float *>(W) + o);
    d[0] = make_float4(v[0], v[1], v[2], v[3]);
    d[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 pk;
    pk.x = pack2<OUT>(v[0], v[1]);
    pk.y = pack2<OUT>(v[2], v[3]);
    pk.z = pack2<OUT>(v[4], v[5]);
    pk.w = pack2<OUT>(v[6], v[7]);
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(W) + o) = pk;
  }
}

hipError_t launch_dequant_w4(const uint8_t *B, const uint16_t *S, const uint16_t *Z, void *W,
                             int n, int k, int group, int act, int out, hipStream_t s) {
  long long runs = static_cast<long long>(n) * k / 8;
  dim3 g(grid_for(runs, 256)), b(256);
#define QG_DQ4(A_, O_) hipLaunchKernelGGL((k_dequant_w4<A_, O_>), g, b, 0, s, B, S, Z, W, n, k, group, runs)
  if (act == kBF16) {
    if (out == QG_FP32) QG_DQ4(kBF16, QG_FP32); else QG_DQ4(kBF16, kBF16);
  } else {
    if (out == QG_FP32) QG_DQ4(kFP16, QG_FP32); else QG_DQ4(kFP16, kFP16);
  }
#undef QG_DQ4
  return hipGetLastError();
}

hipError_t launch_dequant_w8(const int8_t *B, const uint16_t *S, void *W, int n, int k, int group,
                             int act, int out, hipStream_t s) {
  long long runs = static_cast<long long>(n) * k / 8;
  dim3 g(grid_for(runs, 256)), b(256);
#define QG_DQ8(A_, O_) hipLaunchKernelGGL((k_dequant_w8<A_, O_>), g, b, 0, s, B, S, W, n, k, group, runs)
  if (act == kBF16) {
    if (out == QG_FP32) QG_DQ8(kBF16, QG_FP32); else QG_DQ8(kBF16, kBF16);
  } else {
    if (out == QG_FP32) QG_DQ8(kFP16, QG_FP32); else QG_DQ8(kFP16, kFP16);
  }
#undef QG_DQ8
  return hipGetLastError();
}

}  // namespace qg
