// embed.hip -- quantized embedding lookup on gfx950: out[t, :] = the
// dequantized row ids[t] of an int4 or int8 table [vocab, hidden].
//
// vllm-omni cpu_int4.py, CPUInt4EmbeddingMethod: with tied embeddings the
// vocab table and the output head are one quantized tensor; a lookup gathers
// the token's rows, dequantizes them in fp32 with the linear layers' rule and
// casts them to the activation dtype.  The page keeps a second, row-major
// copy of the table for lookups because its GEMM layout cannot address one
// row.  The tiled layouts here can: a row of a 16-channel tile is 16-byte
// slots (int4: 4 per 128-k block; int8: 8 per 64-k block) at fixed offsets,
// so the lookup reads the same bytes the lm_head GEMM streams and one copy
// serves both.  The portable layouts are accepted as well.
//
// One thread per 8 consecutive elements of an output row: one 32-bit word of
// int4 codes or 8 bytes of int8 codes, one scale (and zero), 16 or 32 bytes
// out.  Ids outside [0, vocab) give rows of zeros.
#include "qg_common.hpp"
#include "qg_launch.hpp"

namespace qg {

namespace {

__host__ __device__ inline unsigned grid_of(long long n, int block) {
  return static_cast<unsigned>((n + block - 1) / block);
}

template <int OUT>
__device__ __forceinline__ void store8(void *out, size_t o, const float (&v)[8]) {
  if constexpr (OUT == QG_FP32) {
    f32x4 *d = reinterpret_cast<f32x4 *>(static_cast<float *>(out) + o);
    d[0] = f32x4{v[0], v[1], v[2], v[3]};
    d[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(out) + o) =
        u32x4{pack2<OUT>(v[0], v[1]), pack2<OUT>(v[2], v[3]), pack2<OUT>(v[4], v[5]), pack2<OUT>(v[6], v[7])};
  }
}

// int4: w = (q - 8) * s + z, the product exact in fp32, one rounding (the
// fused form rounds the same single time); then one rounding to OUT.
template <int ACT, int OUT, bool TILED>
__global__ __launch_bounds__(256) void k_embed_w4(const int32_t *__restrict__ ids, int tokens,
                                                  const uint8_t *__restrict__ B,
                                                  const uint16_t *__restrict__ S,
                                                  const uint16_t *__restrict__ Z,
                                                  void *__restrict__ out, int vocab, int hidden,
                                                  int group) {
  const long long r = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = hidden >> 3;
  if (r >= static_cast<long long>(tokens) * per_row) return;
  const int t = static_cast<int>(r / per_row), k0 = static_cast<int>(r % per_row) * 8;
  const int id = ids[t];
  float v[8];
  if (id < 0 || id >= vocab) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
  } else {
    uint32_t word;
    if constexpr (TILED) word = *reinterpret_cast<const uint32_t *>(B + w4_word_offset(id, k0, hidden));
    else word = *reinterpret_cast<const uint32_t *>(B + static_cast<size_t>(id) * (hidden >> 1) + (k0 >> 1));
    const size_t gi = static_cast<size_t>(id) * (hidden / group) + k0 / group;
    const float s = bits_to_f32<ACT>(S[gi]);
    const float z = Z ? bits_to_f32<ACT>(Z[gi]) : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t q = TILED ? w4_tiled_code(word, e) : (word >> (4 * e)) & 0xFu;
      v[e] = __builtin_fmaf(static_cast<float>(static_cast<int>(q) - 8), s, z);
    }
  }
  store8<OUT>(out, static_cast<size_t>(t) * hidden + k0, v);
}

// int8: w = q * s (exact in fp32); group 0 = one scale per row.
template <int ACT, int OUT, bool TILED>
__global__ __launch_bounds__(256) void k_embed_w8(const int32_t *__restrict__ ids, int tokens,
                                                  const int8_t *__restrict__ B,
                                                  const uint16_t *__restrict__ S,
                                                  void *__restrict__ out, int vocab, int hidden,
                                                  int group) {
  const long long r = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = hidden >> 3;
  if (r >= static_cast<long long>(tokens) * per_row) return;
  const int t = static_cast<int>(r / per_row), k0 = static_cast<int>(r % per_row) * 8;
  const int id = ids[t];
  float v[8];
  if (id < 0 || id >= vocab) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
  } else {
    u32x2 run;
    if constexpr (TILED) run = *reinterpret_cast<const u32x2 *>(B + w8_run_offset(id, k0, hidden));
    else run = *reinterpret_cast<const u32x2 *>(B + static_cast<size_t>(id) * hidden + k0);
    const float s = bits_to_f32<ACT>(group > 0 ? S[static_cast<size_t>(id) * (hidden / group) + k0 / group] : S[id]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t byte = ((e < 4 ? run.x : run.y) >> (8 * (e & 3))) & 0xFFu;
      // tiled bytes are offset binary (q + 128); portable ones two's complement
      const int q = TILED ? static_cast<int>(byte) - 128 : static_cast<int>(static_cast<int8_t>(byte));
      v[e] = static_cast<float>(q) * s;
    }
  }
  store8<OUT>(out, static_cast<size_t>(t) * hidden + k0, v);
}

template <int ACT, int OUT>
void embed4(const EmbedArgs &a, hipStream_t s) {
  const long long n = static_cast<long long>(a.tokens) * (a.hidden >> 3);
  const auto *B = static_cast<const uint8_t *>(a.B);
  if (a.tiled)
    hipLaunchKernelGGL((k_embed_w4<ACT, OUT, true>), dim3(grid_of(n, 256)), dim3(256), 0, s, a.ids, a.tokens,
                       B, a.S, a.Z, a.out, a.vocab, a.hidden, a.group);
  else
    hipLaunchKernelGGL((k_embed_w4<ACT, OUT, false>), dim3(grid_of(n, 256)), dim3(256), 0, s, a.ids,
                       a.tokens, B, a.S, a.Z, a.out, a.vocab, a.hidden, a.group);
}

template <int ACT, int OUT>
void embed8(const EmbedArgs &a, hipStream_t s) {
  const long long n = static_cast<long long>(a.tokens) * (a.hidden >> 3);
  const auto *B = static_cast<const int8_t *>(a.B);
  if (a.tiled)
    hipLaunchKernelGGL((k_embed_w8<ACT, OUT, true>), dim3(grid_of(n, 256)), dim3(256), 0, s, a.ids, a.tokens,
                       B, a.S, a.out, a.vocab, a.hidden, a.group);
  else
    hipLaunchKernelGGL((k_embed_w8<ACT, OUT, false>), dim3(grid_of(n, 256)), dim3(256), 0, s, a.ids,
                       a.tokens, B, a.S, a.out, a.vocab, a.hidden, a.group);
}

}  // namespace

hipError_t launch_embed(const EmbedArgs &a, hipStream_t s) {
  const bool f32 = a.out_dt == QG_FP32;
  if (a.bits == 4) {
    if (a.act == kBF16) f32 ? embed4<kBF16, QG_FP32>(a, s) : embed4<kBF16, kBF16>(a, s);
    else f32 ? embed4<kFP16, QG_FP32>(a, s) : embed4<kFP16, kFP16>(a, s);
  } else {
    if (a.act == kBF16) f32 ? embed8<kBF16, QG_FP32>(a, s) : embed8<kBF16, kBF16>(a, s);
    else f32 ? embed8<kFP16, QG_FP32>(a, s) : embed8<kFP16, kFP16>(a, s);
  }
  return hipGetLastError();
}

}  // namespace qg
