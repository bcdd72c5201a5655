// tile_big.hpp -- the large-tile prefill GEMM for gfx950: a 256 x 256 tile of
// C = A . W^T per workgroup, four waves of 128 x 128, one wave per SIMD.
//
// With one wave per SIMD nothing else hides latency, so the kernel pipelines
// explicitly:
//  - A goes from global memory straight into LDS (global_load_lds_dwordx4)
//    one 64-k step ahead of use, into one of two LDS stages;
//  - the packed weight codes (and their scales) are loaded into registers two
//    steps ahead, dequantized by all 256 threads and written into one of two
//    LDS stages while the matrix cores work on the current stage;
//  - operand fragments are double-buffered in registers across the four
//    16-k sub-steps of a step, so the LDS reads of sub-step s + 1 are in
//    flight during the sixteen v_mfma_f32_32x32x16 of sub-step s.
// The 128 x 128 wave tile halves the LDS bytes read per matrix-core
// instruction relative to 64 x 64 tiles (LDS bandwidth limits this part).
//
// LDS rows hold 64 k (128 bytes) plus a 16-byte pad: with a 144-byte stride
// the 16 rows served together by one 16-byte-per-lane access land on 16
// distinct bank groups, and every sub-step / stage offset is a compile-time
// immediate of the LDS instruction (an XOR placement would need a register
// per (stage, sub-step, fragment)).  The stages are separate __shared__
// objects addressed only by constants, so alias analysis can tell the
// direct-to-LDS writes into one stage from the reads of the other.
//
// Rows of A past the problem's end are read from the last valid row (a
// direct-to-LDS load cannot be masked); their output rows are never stored.
#pragma once

#include <type_traits>

#include "tile_gemm.hpp"

namespace qg {

struct BigCfg {
  static constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
  static constexpr int RS = 144;                      // LDS row stride (bytes)
  static constexpr int STAGE = 256 * RS;              // 36864 bytes
  static constexpr int TM = 4, TN = 4;                // 32x32 subtiles per wave
  static constexpr int A_DMA = 9;                     // 1 KiB direct loads per wave per step
};

struct BigLds {
  char *a[2];
  char *b[2];
};

template <int ACT, int WBITS>
__device__ __forceinline__ void tile_gemm_big(const TileProblem &p, int tile_m, int tile_n,
                                              const BigLds &L) {
  using Cfg = BigCfg;
  constexpr int BK = Cfg::BK, RS = Cfg::RS;
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K;
  const int nsteps = K / BK;
  const int row_lo = tile_m * Cfg::BM;
  const int row_last = min(p.M, row_lo + Cfg::BM) - 1;
  const int n0 = tile_n * Cfg::BN;

  // ---- A: 9 direct loads per wave per step, 64 x 16 bytes each, filling
  // the stage linearly: 16-byte slot q holds row q / 9, chunk q % 9 (chunk 8
  // is the pad, loaded from the row's first chunk and never read).
  // 32-bit element offsets keep the address registers few; the host sends
  // problems whose offsets would not fit to the generic tile kernel.
  uint32_t a_off32[Cfg::A_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::A_DMA; ++i) {
    const int q = (wave * Cfg::A_DMA + i) * 64 + lane;
    const int r = q / 9, ch = q % 9;
    const int grow = min(row_lo + r, row_last);
    a_off32[i] = static_cast<uint32_t>(grow) * static_cast<uint32_t>(K) + (ch == 8 ? 0 : ch * 8);
  }
  auto a_issue = [&](int step, char *stage) {
    char *dst = stage + wave * Cfg::A_DMA * 1024;
#pragma unroll
    for (int i = 0; i < Cfg::A_DMA; ++i)
      __builtin_amdgcn_global_load_lds(p.A + a_off32[i] + step * BK,
                                       (__attribute__((address_space(3))) void *)(dst + i * 1024),
                                       16, 0, 0);
  };

  // ---- W: packed codes (and scales) per thread.
  constexpr int NB = (WBITS == 4) ? 4 : 8;   // 8-byte runs per thread per step
  uint32_t b_src[NB];        // byte offsets into the tiled codes
  int b_lds0[NB], b_lds1[NB];
  uint32_t b_sidx[NB];       // scale row offsets
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int idx = tid + c * Cfg::NTHR;
    int l, bi, t = 0;
    if constexpr (WBITS == 4) { l = idx & 63; bi = idx >> 6; }
    else { t = idx & 1; l = (idx >> 1) & 63; bi = idx >> 7; }
    const int nl = l & 15, j = l >> 4;
    const int lrow = bi * 16 + nl;
    const int wrow = n0 + lrow;
    if constexpr (WBITS == 4) {
      b_src[c] = static_cast<uint32_t>(wrow >> 4) * static_cast<uint32_t>(K >> 7) * 1024u + l * 16;
      b_lds0[c] = lrow * RS + j * 16;           // word 2h   -> k-chunk j
      b_lds1[c] = lrow * RS + (4 + j) * 16;     // word 2h+1 -> k-chunk 4 + j
      b_sidx[c] = static_cast<uint32_t>(wrow) * static_cast<uint32_t>(K / p.group);
    } else {
      b_src[c] = static_cast<uint32_t>(wrow >> 4) * static_cast<uint32_t>(K >> 6) * 1024u + l * 16 + t * 8;
      b_lds0[c] = lrow * RS + (4 * t + j) * 16;
      b_lds1[c] = 0;
      b_sidx[c] = 0;
    }
  }
  struct Regs {
    u32x2 b[NB];
    uint16_t s[NB], z[NB];
  };
  auto b_issue = [&](int step, Regs &r) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if constexpr (WBITS == 4) {
        const int kb = step >> 1, h = step & 1;
        r.b[c] = *reinterpret_cast<const u32x2 *>(p.B + b_src[c] + static_cast<uint32_t>(kb) * 1024u + h * 8);
        const uint32_t gi = b_sidx[c] + (step * BK) / p.group;
        r.s[c] = p.S[gi];
        r.z[c] = p.Z[gi];
      } else {
        r.b[c] = *reinterpret_cast<const u32x2 *>(p.B + b_src[c] + static_cast<uint32_t>(step) * 1024u);
      }
    }
  };
  auto b_store = [&](char *Bs, const Regs &r) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if constexpr (WBITS == 4) {
        const float s = bits_to_f32<ACT>(r.s[c]);
        const float z8 = bits_to_f32<ACT>(r.z[c]) - 8.0f * s;
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) = dequant_word_w4<ACT>(r.b[c].x, s, z8);
        *reinterpret_cast<u32x4 *>(Bs + b_lds1[c]) = dequant_word_w4<ACT>(r.b[c].y, s, z8);
      } else {
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) =
            (ACT == kFP16) ? w8_run_to_f16(r.b[c].x, r.b[c].y) : w8_run_to_bf16(r.b[c].x, r.b[c].y);
      }
    }
  };

  // ---- fragments: lane reads row (wave tile row + lane % 32), k-chunk
  // 2 * ks + lane / 32, i.e. a fixed per-lane base plus an immediate.
  const int khalf = lane >> 5;
  const int a_base = (wm * 128 + (lane & 31)) * RS + khalf * 16;
  const int b_base = (wn * 128 + (lane & 31)) * RS + khalf * 16;
  struct Frags {
    u32x4 a[TM], b[TN];
  };
  auto fread = [&](const char *As, const char *Bs, int ks, Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      f.a[i] = *reinterpret_cast<const u32x4 *>(As + a_base + 32 * i * RS + 32 * ks);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      f.b[j] = *reinterpret_cast<const u32x4 *>(Bs + b_base + 32 * j * RS + 32 * ks);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto mma = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<ACT>(f.a[i], f.b[j], acc[i][j]);
  };

  // VMEM instructions this wave issues per step after its A loads of that
  // step: the W loads (codes, scales, zeros) of the step two ahead.  The
  // waits and barriers are written out rather than taken from
  // __syncthreads(), whose workgroup fence would also wait for those W loads
  // (the fence counts the direct-to-LDS loads as pending LDS writes).
  constexpr int VMEM_B = (WBITS == 4) ? 3 * NB : NB;

  // ---- prologue: A step 0 and W steps 0, 1 in flight; W step 0 staged.
  // The empty asm statements with a memory clobber pin the issue order (A
  // loads before W loads), which the explicit vmcnt waits count on.
  Regs r0, r1;
  a_issue(0, L.a[0]);
  asm volatile("" ::: "memory");
  b_issue(0, r0);
  b_issue(min(1, nsteps - 1), r1);
  b_store(L.b[0], r0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VMEM_B) : "memory");

  // ---- one step s (stage I = s % 2): issue A of step s + 1 into A stage
  // 1 - I and the W codes of step s + 2 into `nxt2`; compute on stage I while
  // dequantizing step s + 1 (held in `nxt1`) into W stage 1 - I; wait for this
  // wave's A loads; meet the other waves.  Near the end the issued step is
  // clamped to the last one (the loads are then unused, or rewrite equal
  // bytes into the idle stage).
  auto body = [&](auto Ic, int step, Regs &nxt1, Regs &nxt2) {
    constexpr int I = decltype(Ic)::value;
    char *As = L.a[I];
    char *Bs = L.b[I];
    a_issue(min(step + 1, nsteps - 1), L.a[1 - I]);
    asm volatile("" ::: "memory");
    b_issue(min(step + 2, nsteps - 1), nxt2);
    __builtin_amdgcn_sched_barrier(0);
    Frags f0, f1;
    fread(As, Bs, 0, f0);
    fread(As, Bs, 1, f1);
    mma(f0);
    b_store(L.b[1 - I], nxt1);
    fread(As, Bs, 2, f0);
    mma(f1);
    fread(As, Bs, 3, f1);
    mma(f0);
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VMEM_B) : "memory");
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  int step = 0;
  for (; step + 2 <= nsteps; step += 2) {
    body(I0{}, step, r1, r0);
    body(I1{}, step + 1, r0, r1);
  }
  if (step < nsteps) body(I0{}, step, r1, r0);

  // ---- epilogue
  const int col_in = lane & 31;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * 128 + 32 * j + col_in;
    float cs = 1.0f, cb = 0.0f;
    if constexpr (WBITS == 8) cs = bits_to_f32<ACT>(p.S[col]);
    if (p.bias) cb = bits_to_f32_dyn(p.bias[col], p.bias_dt);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = row_lo + wm * 128 + 32 * i + 8 * (v >> 2) + 4 * khalf + (v & 3);
        if (r <= row_last) {
          float val = acc[i][j][v];
          if constexpr (WBITS == 8) val *= cs;
          val += cb;
          p.C[static_cast<size_t>(r) * p.N + col] = f32_to_bits<ACT>(val);
        }
      }
  }
}

}  // namespace qg
