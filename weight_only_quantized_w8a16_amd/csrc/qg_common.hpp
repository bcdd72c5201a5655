// qg_common.hpp -- device helpers shared by the gfx950 kernels of libqgemm.
//
// Fragment types for the CDNA4 matrix instructions, 16-bit float bit
// conversions, and the tiled weight layout address arithmetic documented in
// include/qgemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemm.h"

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Activation dtype codes (match qg_dtype).
constexpr int kBF16 = QG_BF16;
constexpr int kFP16 = QG_FP16;

// ---------------------------------------------------------------------------
// 16-bit float <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (the hardware conversion under the default round mode).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
template <int DT>
__device__ __forceinline__ float bits_to_f32(uint16_t h) {
  if constexpr (DT == kFP16) return f16_bits_to_f32(h);
  else return bf16_bits_to_f32(h);
}
__device__ __forceinline__ float bits_to_f32_dyn(uint16_t h, int dt) {
  return dt == kFP16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
}
template <int DT>
__device__ __forceinline__ uint16_t f32_to_bits(float x) {
  if constexpr (DT == kFP16) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  else return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
// Two fp32 values -> packed pair of 16-bit floats (low half = a).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == kFP16) {
    f16x2 v = __builtin_convertvector(f32x2{a, b}, f16x2);
    return __builtin_bit_cast(uint32_t, v);
  } else {
    bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
  }
}

// ---------------------------------------------------------------------------
// Tiled int4 layout (see include/qgemm.h): 1 KiB per (16 n) x (128 k) block,
// 64 lane slots of 16 bytes, 32-bit word t of slot (j, nl) holding the codes
// k = 128*kb + 32*t + 8*j + e, even e in the low half-word.
// ---------------------------------------------------------------------------
// Word of the portable row (8 consecutive codes, code e in nibble e) ->
// tiled word (code e in nibble e/2 for even e, 4 + e/2 for odd e).
__device__ __forceinline__ uint32_t w4_to_tiled_word(uint32_t v) {
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t nib = (v >> (4 * e)) & 0xFu;
    int pos = (e & 1) ? 4 + (e >> 1) : (e >> 1);
    out |= nib << (4 * pos);
  }
  return out;
}
__device__ __forceinline__ uint32_t w4_from_tiled_word(uint32_t v) {
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int pos = (e & 1) ? 4 + (e >> 1) : (e >> 1);
    out |= ((v >> (4 * pos)) & 0xFu) << (4 * e);
  }
  return out;
}

// Code e (0..7) of a tiled word.
__device__ __forceinline__ uint32_t w4_tiled_code(uint32_t v, int e) {
  int pos = (e & 1) ? 4 + (e >> 1) : (e >> 1);
  return (v >> (4 * pos)) & 0xFu;
}

// Byte offset of the 32-bit word holding codes (n, k0..k0+7), k0 % 8 == 0.
__device__ __forceinline__ size_t w4_word_offset(int n, int k0, int K) {
  int nt = n >> 4, nl = n & 15, kb = k0 >> 7, r = k0 & 127;
  int t = r >> 5, j = (r >> 3) & 3;
  return (static_cast<size_t>(nt) * (K >> 7) + kb) * 1024u + (16 * j + nl) * 16 + t * 4;
}

// Tiled int8 layout: 1 KiB per (16 n) x (64 k) block; slot (j, nl) holds
// k = 64*kb + 32*t + 8*j + e at byte t*8 + e, stored as q ^ 0x80.
__device__ __forceinline__ size_t w8_run_offset(int n, int k0, int K) {
  int nt = n >> 4, nl = n & 15, kb = k0 >> 6, r = k0 & 63;
  int t = r >> 5, j = (r >> 3) & 3;
  return (static_cast<size_t>(nt) * (K >> 6) + kb) * 1024u + (16 * j + nl) * 16 + t * 8;
}

// ---------------------------------------------------------------------------
// Exact small-integer operands for the matrix cores.
// A tiled int4 word -> 8 values (128 + q) as bf16, or (1024 + q) as fp16,
// in k order: one AND-OR per pair, no rounding anywhere.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ u32x4 w4_word_to_operand(uint32_t w) {
  constexpr uint32_t magic = (DT == kFP16) ? 0x64006400u : 0x43004300u;
  u32x4 r;
  r.x = (w & 0x000F000Fu) | magic;
  r.y = ((w >> 4) & 0x000F000Fu) | magic;
  r.z = ((w >> 8) & 0x000F000Fu) | magic;
  r.w = ((w >> 12) & 0x000F000Fu) | magic;
  return r;
}
// The same with the mask and the exponent pattern in registers (W4Consts,
// made once per kernel outside its loops, opaque to the optimizer): with
// both as literals the compiler emits a separate AND and OR per pair (a
// three-operand instruction on gfx9 takes no literal), with them in
// registers one v_and_or_b32 -- 7 instead of 11 VALU instructions per word,
// for the VALU-heavy streaming decode kernel.
struct W4Consts {
  uint32_t magic, mask;
};
template <int DT>
__device__ __forceinline__ W4Consts w4_consts() {
  W4Consts c{(DT == kFP16) ? 0x64006400u : 0x43004300u, 0x000F000Fu};
  asm volatile("" : "+v"(c.magic));
  asm volatile("" : "+s"(c.mask));
  return c;
}
template <int DT>
__device__ __forceinline__ u32x4 w4_word_to_operand(uint32_t w, W4Consts c) {
  u32x4 r;
  r.x = (w & c.mask) | c.magic;
  r.y = ((w >> 4) & c.mask) | c.magic;
  r.z = ((w >> 8) & c.mask) | c.magic;
  r.w = ((w >> 12) & c.mask) | c.magic;
  return r;
}
// silu(g) * u = g / (1 + exp(-g)) * u with the hardware reciprocal (about
// one ulp of fp32) instead of an IEEE-rounded division, whose scaling and
// fix-up steps cost about ten instructions per value; the result is rounded
// to the 16-bit activation type right after.  exp(-g) overflowing to +inf
// gives 0 * g, the limit.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}
// Offset that w4_word_to_operand adds to each code.
template <int DT>
constexpr float w4_operand_offset() { return DT == kFP16 ? 1024.0f : 128.0f; }

// Two offset-binary int8 bytes (u = q + 128) -> fp16 pair (1024 + u) via a
// byte permute against 0x64, then an exact fp16 subtract of 1152 gives q.
__device__ __forceinline__ uint32_t w8_pair_to_f16(uint32_t w, uint32_t sel) {
  uint32_t p = __builtin_amdgcn_perm(0x64646464u, w, sel);
  f16x2 v = __builtin_bit_cast(f16x2, p);
  v = v - f16x2{(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, v);
}
// 8 offset-binary bytes (two words) -> 8 exact fp16 values q.
__device__ __forceinline__ u32x4 w8_run_to_f16(uint32_t lo, uint32_t hi) {
  // perm selector: byte i of the result; 0..3 pick from the second operand
  // (w), 4..7 from the first (0x64 everywhere).
  constexpr uint32_t sel01 = 0x04010400u;  // [w.b0, 0x64, w.b1, 0x64]
  constexpr uint32_t sel23 = 0x04030402u;  // [w.b2, 0x64, w.b3, 0x64]
  u32x4 r;
  r.x = w8_pair_to_f16(lo, sel01);
  r.y = w8_pair_to_f16(lo, sel23);
  r.z = w8_pair_to_f16(hi, sel01);
  r.w = w8_pair_to_f16(hi, sel23);
  return r;
}
// 8 offset-binary bytes -> 8 exact bf16 values q (through exact fp32).
__device__ __forceinline__ u32x4 w8_run_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  uint32_t ws[2] = {lo, hi};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float f0 = static_cast<float>(static_cast<int>((ws[h] >> 0) & 0xFFu) - 128);
    float f1 = static_cast<float>(static_cast<int>((ws[h] >> 8) & 0xFFu) - 128);
    float f2 = static_cast<float>(static_cast<int>((ws[h] >> 16) & 0xFFu) - 128);
    float f3 = static_cast<float>(static_cast<int>((ws[h] >> 24) & 0xFFu) - 128);
    // |q| <= 128 has at most 8 significant bits: the bf16 narrowing is exact.
    r[2 * h] = pack2<kBF16>(f0, f1);
    r[2 * h + 1] = pack2<kBF16>(f2, f3);
  }
  return r;
}

// ---------------------------------------------------------------------------
// Matrix-core wrappers (gfx950).
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == kFP16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == kFP16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 1.0 in both halves.
template <int DT>
constexpr uint32_t one_pair() { return DT == kFP16 ? 0x3C003C00u : 0x3F803F80u; }

}  // namespace qg
