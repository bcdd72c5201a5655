// tile_big.hpp -- the direct-load prefill GEMM tile for gfx950: C = A . W^T
// for one BM x BN output tile per workgroup (BM 64, 128 or 256; BN 128 or
// 256), WM x WN waves, each wave a (BM / WM) x (BN / WN) block of 32 x 32
// accumulators.
//
// Per 64-k step:
//  - A goes from global memory into LDS with buffer_load_dwordx4 ... lds,
//    one step ahead of use, into one of two LDS stages (no trip through
//    VGPRs, so no registers, address arithmetic or LDS store instructions
//    for it);
//  - the packed weight codes are loaded into registers two steps ahead,
//    dequantized by every thread and written into one of two LDS stages
//    while the matrix cores work on the current stage;
//  - the int4 scales and zeros come through LDS as well: a window holds 8
//    groups of the tile's BN channels (16 bytes of each row of the scale and
//    zero matrices, read with 4-byte direct loads, one 2 KiB part per step),
//    so each row's scales cost one cache-line visit per 8 groups instead of
//    a 16-line gather per group;
//  - every wave then waits for its own direct loads and meets the others at
//    one barrier.
//
// LDS placement: a stage holds BM (A) or BN (W) rows of 64 k (128 bytes),
// the 16-byte chunk c of row r at chunk c ^ ((r / 2) % 8).  A 16-lane group
// reading one chunk of 16 consecutive rows then touches 16 distinct 16-byte
// bank groups of the 256-byte bank space.  A direct load writes 64
// consecutive 16-byte slots, so the swizzle is applied on the source side:
// slot (r, c') is loaded from the row's chunk c' ^ ((r / 2) % 8).
//
// Rows of A past the problem's end are read from the last valid row (a
// direct-to-LDS load cannot be masked); their output rows are never stored.
// All loads go through buffer resources with 32-bit offsets: the host routes
// problems with M * K or the code bytes at or above 2^31 elsewhere.
#pragma once

#include <type_traits>

#include "tile_gemm.hpp"

namespace qg {

template <int WM_, int WN_, int BN_ = 256, int BM_ = 256>
struct DmaCfg {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int NTHR = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 accumulators per wave
  static constexpr int STAGE_A = BM * 128;             // bytes per A stage
  static constexpr int STAGE_B = BN * 128;             // bytes per W stage
  static constexpr int A_DMA = BM * 8 / NTHR;          // direct loads per thread per step
  static constexpr int NB4 = BN * 4 / NTHR;            // int4: 8-byte code runs per thread
  static constexpr int NB8 = BN * 8 / NTHR;            // int8: 8-byte code runs per thread
  static constexpr int SC_WIN = 2 * BN * 16;           // bytes per scale/zero window
  static constexpr int SC_PARTS = BN / 64;             // 2 KiB parts per window
  static constexpr int SC_DMA = 512 / NTHR;            // 4-byte window loads per thread per step
  static_assert(BN == 128 || BN == 256, "tile width");
  static_assert(BM % 64 == 0 && WTM % 32 == 0, "tile height");
  static_assert(A_DMA >= 1 && NB4 >= 1 && SC_DMA >= 1, "thread count");
};

struct DmaLds {
  char *a[2];
  char *b[2];
  char *sc;   // two scale/zero windows of DmaCfg::SC_WIN bytes
  char *ep;   // dense tiles: the tile's bias, then its int8 channel scales (2 x BN x 2 bytes)
};

__device__ __forceinline__ int dswz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// MODE (tile_gemm.hpp): kDense; kMoeFc1 -- rows of one expert's tile, the
// activation rows gathered through row_src, the 256 weight rows being 128
// gate and the matching 128 up rows of the expert (wave column block wn
// holds gate rows 32 wn .. 32 wn + 31 of the tile's 128 outputs, then the
// same up rows), output silu(gate) * up; kMoeFc2 -- rows of one expert's
// tile, contiguous.
// GS8 (int8 only): one scale per (channel, K-group), brought through the
// same LDS windows as the int4 scales (the zero half of each window holds a
// second copy of the scales, unused) and applied while dequantizing.
// SPLIT: a dense split-K launch (TileProblem::part, kseg); `slice` is this
// workgroup's K slice.  With scale windows kseg is a multiple of a window's
// steps, so a slice starts on a window boundary.  Without SPLIT the kernel
// runs all of K and the slice code is not compiled in.
// PC (int4 only): one scale and zero per channel (group = K), read once per
// run into registers instead of through the LDS windows.
template <class Cfg, int ACT, int WBITS, int MODE = kDense, bool GS8 = false, bool SPLIT = false,
          bool PC = false>
__device__ __forceinline__ void tile_gemm_dma(const TileProblem &p, int tile_m, int tile_n,
                                              const DmaLds &L, int slice = 0) {
  constexpr int BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN, NTHR = Cfg::NTHR;
  static_assert(MODE == kDense || WBITS == 4, "MoE experts are int4");
  static_assert(!GS8 || WBITS == 8, "group scales without zeros: int8");
  static_assert(!PC || (WBITS == 4 && MODE == kDense), "per-channel int4: dense");
  constexpr bool kWin = (WBITS == 4 && !PC) || GS8;   // scales through the LDS windows
  static_assert(MODE != kMoeFc1 || Cfg::BN == 256, "fc1 pairs 128 gate with 128 up rows");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int K = p.K;
  static_assert(!SPLIT || MODE == kDense, "split-K: dense problems");
  const int s0 = SPLIT ? slice * p.kseg : 0;                    // steps [s0, s1)
  const int s1 = SPLIT ? min(K / BK, s0 + p.kseg) : K / BK;
  int row_lo, row_last;
  [[maybe_unused]] int expert = 0;
  const uint8_t *Bb = p.B;
  const uint16_t *Sb = p.S, *Zb = GS8 ? p.S : p.Z;
  uint32_t b_bytes, s_bytes;     // buffer extents (one expert for MoE)
  if constexpr (MODE == kDense) {
    row_lo = tile_m * Cfg::BM;
    row_last = min(p.M, row_lo + Cfg::BM) - 1;
    b_bytes = static_cast<uint32_t>(static_cast<uint64_t>(p.N) * K * WBITS / 8);
    s_bytes = kWin ? static_cast<uint32_t>(static_cast<uint64_t>(p.N) * (K / p.group) * 2) : 0u;
  } else {
    const MoeTile t = p.tiles[tile_m];
    expert = t.expert;
    row_lo = t.row0;
    row_last = t.row1 - 1;
    Bb += static_cast<size_t>(t.expert) * p.b_expert_stride;
    Sb += static_cast<size_t>(t.expert) * p.s_expert_stride;
    Zb += static_cast<size_t>(t.expert) * p.s_expert_stride;
    b_bytes = static_cast<uint32_t>(p.b_expert_stride);
    s_bytes = static_cast<uint32_t>(p.s_expert_stride * 2);
  }
  const int n0 = (MODE == kMoeFc1) ? tile_n * (Cfg::BN / 2) : tile_n * Cfg::BN;
  // Weight row of LDS row `lrow` (0 .. BN - 1).
  auto wrow_of = [&](int lrow) {
    if constexpr (MODE == kMoeFc1)
      return (((lrow >> 5) & 1) ? p.N : 0) + n0 + 32 * (lrow >> 6) + (lrow & 31);
    else
      return n0 + lrow;
  };

  // Buffer resources: 32-bit per-lane offsets, the step's offset in an SGPR.
  // (A flat/global direct-to-LDS load would also be taken by the wait-count
  // pass as a pending LDS access, and every later wait would become a full
  // drain.)
  constexpr int kRsrcFlags = 0x00020000;
  const uint32_t a_bytes = static_cast<uint32_t>(static_cast<uint64_t>(p.a_rows) * K * 2);
  const auto rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.A), 0, static_cast<int>(a_bytes), kRsrcFlags);
  const auto rB = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(Bb), 0, static_cast<int>(b_bytes), kRsrcFlags);
  [[maybe_unused]] const auto rS =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(Sb), 0, static_cast<int>(s_bytes), kRsrcFlags);
  // No zeros (scale-only int4): an empty resource, whose loads return 0.
  [[maybe_unused]] const auto rZ = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(Zb), 0, Zb ? static_cast<int>(s_bytes) : 0, kRsrcFlags);

  // ---- epilogue constants: the tile's BN bias values and (per-channel int8)
  // BN channel scales, 16-bit each, come into L.ep by 4-byte direct loads in
  // the prologue (waves 0 .. BN / 128 - 1 the bias, the next ones the
  // scales, 256 bytes a wave), so the epilogue reads them from LDS instead of
  // waiting on 32 two-byte global loads per lane (measured at M = 512,
  // N = 131072: 4.2k of the tile's 112k cycles).  A pointer that is not
  // 4-byte aligned keeps the global loads.
  constexpr bool kEpi = MODE == kDense && !SPLIT;
  constexpr bool kColScale = WBITS == 8 && !GS8;
  constexpr int kEpWaves = Cfg::BN / 128;
  [[maybe_unused]] const bool bias_lds =
      kEpi && p.bias && (reinterpret_cast<uintptr_t>(p.bias) & 3) == 0;
  [[maybe_unused]] const bool cs_lds = kEpi && kColScale && (reinterpret_cast<uintptr_t>(p.S) & 3) == 0;
  auto ep_issue = [&] {
    if constexpr (kEpi) {
      const bool scale_wave = wave >= kEpWaves;
      const int part = scale_wave ? wave - kEpWaves : wave;
      if (wave < 2 * kEpWaves && (scale_wave ? cs_lds : bias_lds)) {
        const auto r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(scale_wave ? p.S : p.bias), 0,
            static_cast<int>(static_cast<uint32_t>(p.N) * 2u), kRsrcFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void *)(L.ep + wave * 256), 4, lane * 4,
            (n0 + part * 128) * 2, 0, 0);
      }
    }
  };

  // ---- A: slot q = (wave * A_DMA + i) * 64 + lane of a stage is row q / 8,
  // placed chunk q % 8; it holds the row's chunk (q % 8) ^ ((row / 2) % 8).
  uint32_t a_voff[Cfg::A_DMA];   // bytes
#pragma unroll
  for (int i = 0; i < Cfg::A_DMA; ++i) {
    const int q = (wave * Cfg::A_DMA + i) * 64 + lane;
    const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    int grow = min(row_lo + r, row_last);
    if constexpr (MODE == kMoeFc1) grow = p.row_src[grow];
    a_voff[i] = (static_cast<uint32_t>(grow) * static_cast<uint32_t>(K) + c * 8) * 2u;
  }
  auto a_issue = [&](int step, char *stage) {
    char *dst = stage + wave * Cfg::A_DMA * 1024;
#pragma unroll
    for (int i = 0; i < Cfg::A_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rA, (__attribute__((address_space(3))) void *)(dst + i * 1024), 16, a_voff[i], step * BK * 2, 0, 0);
  };

  // ---- W: packed codes per thread.
  constexpr int NB = (WBITS == 4) ? Cfg::NB4 : Cfg::NB8;
  uint32_t b_src[NB];        // byte offsets into the tiled codes
  int b_lds0[NB], b_lds1[NB];
  int b_sc[NB];              // scale-window offsets of the runs' rows
  [[maybe_unused]] int b_wrow[NB];   // weight rows of the runs (per-channel scales)
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int idx = tid + c * NTHR;
    int l, bi, t = 0;
    if constexpr (WBITS == 4) { l = idx & 63; bi = idx >> 6; }
    else { t = idx & 1; l = (idx >> 1) & 63; bi = idx >> 7; }
    const int nl = l & 15, j = l >> 4;
    const int lrow = bi * 16 + nl;
    const int wrow = wrow_of(lrow);
    b_wrow[c] = wrow;
    if constexpr (WBITS == 4) {
      b_src[c] = static_cast<uint32_t>(wrow >> 4) * static_cast<uint32_t>(K >> 7) * 1024u + l * 16;
      b_lds0[c] = dswz(lrow, j);          // word 2h   -> k-chunk j
      b_lds1[c] = dswz(lrow, 4 + j);      // word 2h+1 -> k-chunk 4 + j
      b_sc[c] = lrow * 16;
    } else {
      b_src[c] = static_cast<uint32_t>(wrow >> 4) * static_cast<uint32_t>(K >> 6) * 1024u + l * 16 + t * 8;
      b_lds0[c] = dswz(lrow, 4 * t + j);
      b_lds1[c] = 0;
      b_sc[c] = GS8 ? lrow * 16 : 0;
    }
  }
  struct Regs {
    u32x2 b[NB];
  };
  auto b_issue = [&](int step, Regs &r) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if constexpr (WBITS == 4) {
        const int kb = step >> 1, h = step & 1;
        r.b[c] = __builtin_amdgcn_raw_buffer_load_b64(rB, b_src[c], kb * 1024 + h * 8, 0);
      } else {
        r.b[c] = __builtin_amdgcn_raw_buffer_load_b64(rB, b_src[c], step * 1024, 0);
      }
    }
  };

  // ---- int4 scale/zero windows.  Window w holds groups 8w .. 8w + 7 of the
  // tile's BN rows: byte (c * BN + row) * 16 + 2 * (group % 8), component c
  // 0 the scales, 1 the zeros; windows alternate between two buffers.  Step
  // u uses group u / spg (spg = group_size / 64 steps per group).  A direct
  // load writes 4 bytes per lane (two groups), so a window is BN / 64 parts
  // of 2 KiB; part t, slot = wave * SC_DMA + i covers rows
  // 128 (t % (BN / 128)) + 16 slot + lane / 4, groups 2 (lane % 4) + {0, 1},
  // of component t / (BN / 128).  At the top of step s, before any new
  // direct load, each thread reads the scales of step s + 1 (dequantized in
  // step s) from LDS; then part (s + 1) % (BN / 64) of window
  // (s + 1) / (8 spg) + 1 is issued (every part at least twice per window,
  // the repeats rewriting equal bytes).  A window is complete one step
  // before its first use, and its buffer was last read one step before its
  // first part lands.  Windows past the last group read other rows or (past
  // the end of the matrices) zeros; they are never used.
  [[maybe_unused]] const int kg = K / p.group;
  [[maybe_unused]] const int spg_lg = (p.group == 128) ? 1 : 0;
  uint32_t sc_voff[Cfg::SC_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::SC_DMA; ++i) {
    const int slot = wave * Cfg::SC_DMA + i;
    sc_voff[i] = (static_cast<uint32_t>(wrow_of(slot * 16 + (lane >> 2))) * static_cast<uint32_t>(kg) + (lane & 3) * 2) * 2u;
  }
  // Rows 128 .. 255 of a 256-row tile are weight rows 128 (fc1: 64) further on.
  constexpr int kHalfRows = (MODE == kMoeFc1) ? 64 : 128;
  constexpr int PPC = Cfg::BN / 128;   // parts per component
  auto sc_issue = [&](int t, int w) {
    if constexpr (kWin) {
      const int soff = (t % PPC) * kHalfRows * kg * 2 + w * 16;
      char *dst = L.sc + (w & 1) * Cfg::SC_WIN + (t * 8 + wave * Cfg::SC_DMA) * 256;
#pragma unroll
      for (int i = 0; i < Cfg::SC_DMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(t >= PPC ? rZ : rS,
                                                 (__attribute__((address_space(3))) void *)(dst + i * 256), 4,
                                                 sc_voff[i], soff, 0, 0);
    }
  };
  struct ScaleRegs {
    uint16_t s[NB], z[NB];
  };
  [[maybe_unused]] ScaleRegs pcv;   // per-channel: fixed for the whole K loop
  if constexpr (PC) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      pcv.s[c] = p.S[b_wrow[c]];
      pcv.z[c] = p.Z ? p.Z[b_wrow[c]] : uint16_t(0);
    }
  }
  auto sc_read = [&](int u, ScaleRegs &v) {
    if constexpr (PC) v = pcv;
    if constexpr (kWin) {
      const int gi = u >> spg_lg;
      const char *win = L.sc + ((gi >> 3) & 1) * Cfg::SC_WIN + (gi & 7) * 2;
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        v.s[c] = *reinterpret_cast<const uint16_t *>(win + b_sc[c]);
        v.z[c] = *reinterpret_cast<const uint16_t *>(win + Cfg::BN * 16 + b_sc[c]);
      }
    }
  };
  auto b_store = [&](char *Bs, const Regs &r, const ScaleRegs &v) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if constexpr (WBITS == 4) {
        const float s = bits_to_f32<ACT>(v.s[c]);
        const float z8 = bits_to_f32<ACT>(v.z[c]) - 8.0f * s;
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) = dequant_word_w4<ACT>(r.b[c].x, s, z8);
        *reinterpret_cast<u32x4 *>(Bs + b_lds1[c]) = dequant_word_w4<ACT>(r.b[c].y, s, z8);
      } else if constexpr (GS8) {
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) =
            dequant_run_w8<ACT>(r.b[c].x, r.b[c].y, bits_to_f32<ACT>(v.s[c]));
      } else {
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) =
            (ACT == kFP16) ? w8_run_to_f16(r.b[c].x, r.b[c].y) : w8_run_to_bf16(r.b[c].x, r.b[c].y);
      }
    }
  };

  // ---- fragments: the tile's 32-row blocks are dealt out to the WM wave rows
  // in turn (block b to wave row b % WM, as its block b / WM), so a partly
  // filled expert tile gives every wave row about the same number of filled
  // blocks.  Lane reads row 32 (i WM + wm) + lane % 32, chunk 2 ks + lane / 32,
  // placed at that ^ ((lane / 2) % 8) (the block offset leaves (row / 2) % 8
  // unchanged).  One address per ks; i and the stage are immediates.
  const int khalf = lane >> 5;
  const int g = khalf ^ ((lane >> 1) & 7);
  int a_addr[4], b_addr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    a_addr[ks] = (wm * 32 + (lane & 31)) * 128 + (((2 * ks) ^ g) << 4);
    b_addr[ks] = (wn * Cfg::WTN + (lane & 31)) * 128 + (((2 * ks) ^ g) << 4);
  }
  struct Frags {
    u32x4 a[TM], b[TN];
  };
  auto fread = [&](auto NAc, const char *As, const char *Bs, int ks, Frags &f) {
#pragma unroll
    for (int i = 0; i < decltype(NAc)::value; ++i)
      f.a[i] = *reinterpret_cast<const u32x4 *>(As + a_addr[ks] + Cfg::WM * 4096 * i);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const u32x4 *>(Bs + b_addr[ks] + 4096 * j);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // The weights are the row operand and the activations the column
  // operand, so acc[i][j] holds C^T: a lane keeps one row of C (activation
  // row 32 i + lane % 32) and 16 of its columns, four consecutive ones per
  // group of four values -- which the epilogue stores as 8-byte pieces.
  auto mma = [&](auto NAc, const Frags &f) {
#pragma unroll
    for (int i = 0; i < decltype(NAc)::value; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<ACT>(f.b[j], f.a[i], acc[i][j]);
  };

  // VMEM instructions a thread issues per step after its direct loads: the
  // W code loads of the step two ahead.  The wait before each barrier leaves
  // exactly those in flight.  It is a compiler builtin (not inline asm), so
  // the wait-count pass knows what it covers and adds no waits of its own
  // for the LDS data read after the barrier.
  constexpr int VMEM_B = NB;
  static_assert(VMEM_B < 16, "vmcnt field");
  constexpr int WAIT = VMEM_B | (7 << 4);                    // vmcnt(VMEM_B) lgkmcnt(0)
  constexpr int WAIT_ALL_BUT_2B = (2 * VMEM_B < 16 ? 2 * VMEM_B : 15) | (7 << 4);
  auto barrier = [&] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- prologue: scale window 0 and part 0 of window 1, A of step 0, W
  // codes of steps 0 and 1; once the direct loads have landed everywhere,
  // dequantize step 0.  The empty asm statements with a memory clobber keep
  // the direct loads ahead of the code loads, which the waits count on.
  Regs r0, r1;
  ScaleRegs sv;
  const int w0 = s0 >> (3 + spg_lg);   // first scale window
#pragma unroll
  for (int t = 0; t < Cfg::SC_PARTS; ++t) sc_issue(t, w0);
  sc_issue(0, w0 + 1);
  ep_issue();
  a_issue(s0, L.a[0]);
  asm volatile("" ::: "memory");
  b_issue(s0, r0);
  b_issue(min(s0 + 1, s1 - 1), r1);
  __builtin_amdgcn_s_waitcnt(WAIT_ALL_BUT_2B);
  barrier();
  sc_read(s0, sv);
  b_store(L.b[0], r0, sv);
  __builtin_amdgcn_s_waitcnt(WAIT);
  barrier();

  // ---- step s on stage I = s % 2: read the scales of step s + 1; issue the
  // next scale-window part, A of step s + 1 into A stage 1 - I and W of step
  // s + 2 into `nxt2`; run the matrix cores on stage I while dequantizing
  // step s + 1 (`nxt1`) into W stage 1 - I.  Stage 1 - I was last read in
  // step s - 1, before the barrier that ended it.  Near the end the issued
  // step is clamped to the last one (the loads are then unused, or rewrite
  // equal bytes into the idle stage).
  auto body = [&](auto NAc, auto Ic, int step, Regs &nxt1, Regs &nxt2) {
    constexpr int I = decltype(Ic)::value;
    constexpr int NA = decltype(NAc)::value;
    char *As = L.a[I];
    char *Bs = L.b[I];
    ScaleRegs v;
    sc_read(step + 1, v);
    asm volatile("" ::: "memory");
    sc_issue((step + 1) % Cfg::SC_PARTS, ((step + 1) >> (3 + spg_lg)) + 1);
    a_issue(min(step + 1, s1 - 1), L.a[1 - I]);
    asm volatile("" ::: "memory");
    b_issue(min(step + 2, s1 - 1), nxt2);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NA > 0) {
      Frags f0, f1;
      fread(NAc, As, Bs, 0, f0);
      fread(NAc, As, Bs, 1, f1);
      mma(NAc, f0);
      b_store(L.b[1 - I], nxt1, v);
      fread(NAc, As, Bs, 2, f0);
      mma(NAc, f1);
      fread(NAc, As, Bs, 3, f1);
      mma(NAc, f0);
      mma(NAc, f1);
      // Keep the fragment reads one sub-step ahead of the matrix cores (the
      // scheduler would otherwise sink each sub-step's reads down to their
      // first use and expose the LDS latency four times per step).
      constexpr int NR = NA + TN, NM = NA * TN;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NR, 0);   // reads, sub-steps 0, 1
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);       // MFMA, sub-step 0
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);       // reads, sub-step 2
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);       // MFMA, sub-step 1
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);       // reads, sub-step 3
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);       // MFMA, sub-step 2
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);       // MFMA, sub-step 3
    } else {
      b_store(L.b[1 - I], nxt1, v);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(WAIT);
    barrier();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  auto main_loop = [&](auto NAc) {
    int step = s0;
    for (; step + 2 <= s1; step += 2) {
      body(NAc, I0{}, step, r1, r0);
      body(NAc, I1{}, step + 1, r0, r1);
    }
    if (step < s1) body(NAc, I0{}, step, r1, r0);
  };
  if constexpr (MODE == kDense) {
    main_loop(std::integral_constant<int, TM>{});
  } else {
    // An expert tile is mostly partly filled: a wave skips the fragment
    // reads and matrix-core work of its 32-row blocks that hold no rows
    // (it still loads and dequantizes its share and meets every barrier).
    // With the blocks dealt out in turn, a 192-row expert gives both wave
    // rows three blocks (in contiguous halves: four and two).
    const int blocks = (row_last - row_lo + 32) >> 5;      // 32-row blocks holding rows
    const int mine = blocks > wm ? (blocks - wm + Cfg::WM - 1) / Cfg::WM : 0;
    const int na = __builtin_amdgcn_readfirstlane(min(TM, mine));
    static_assert(TM == 4, "expert tiles: four 32-row blocks per wave");
    if (na == 4) main_loop(std::integral_constant<int, 4>{});
    else if (na == 3) main_loop(std::integral_constant<int, 3>{});
    else if (na == 2) main_loop(std::integral_constant<int, 2>{});
    else if (na == 1) main_loop(std::integral_constant<int, 1>{});
    else main_loop(std::integral_constant<int, 0>{});
  }

  // ---- epilogue: value v of acc[i][j] is C[row][col], row = 32 (i WM + wm)
  // + lane % 32, col = wave tile column + 32 j + 8 (v / 4) +
  // 4 (lane / 32) + v % 4.  Per i, each wave stages its 32 x 64 block in LDS
  // (8-byte pieces, 144-byte rows) and stores it as 16-byte row pieces, so
  // every store instruction writes whole 128-byte lines (nontemporal: the
  // output is not read again by this kernel; measured 1-3 % faster).  Four waves share
  // one stage (A or W, whichever is large enough); all stages are free: the
  // last step ended with a barrier after every wave's last read.
  if constexpr (SPLIT) {
    {   // split-K slice: the raw fp32 partial sums, 4 columns per store
      float *dst = p.part + static_cast<size_t>(slice) * p.M * p.N;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = row_lo + 32 * (i * Cfg::WM + wm) + (lane & 31);
        if (r > row_last) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n0 + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf;
            *reinterpret_cast<f32x4 *>(dst + static_cast<size_t>(r) * p.N + col) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          }
      }
      return;
    }
  }
  static_assert(Cfg::WTN == 64 && Cfg::NTHR == 512, "epilogue staging assumes 8 waves, 64 columns each");
  constexpr bool kStageInA = Cfg::STAGE_A >= 4 * 32 * 144;
  static_assert(kStageInA || Cfg::STAGE_B >= 4 * 32 * 144, "no LDS stage holds four 32 x 64 blocks");
  char *stg = (kStageInA ? ((wave >> 2) ? L.a[1] : L.a[0]) : ((wave >> 2) ? L.b[1] : L.b[0])) +
              (wave & 3) * (32 * 144);
  const int row_in = lane & 31;
  if constexpr (MODE == kMoeFc1) {
    // acc[i][0] is gate, acc[i][1] up, of output columns
    // n0 + 32 wn + 8 (v / 4) + 4 (lane / 32) + v % 4; 32 x 32 blocks staged
    // in 80-byte rows.  The expert's fc1 biases (gate row col, up row N + col)
    // are added before the activation.
    float bg[4][4], bu[4][4];
    const uint16_t *b1 = p.bias ? p.bias + static_cast<size_t>(expert) * p.w_rows : nullptr;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = n0 + 32 * wn + 8 * q + 4 * khalf + e;
        bg[q][e] = b1 ? bits_to_f32<ACT>(b1[col]) : 0.0f;
        bu[q][e] = b1 ? bits_to_f32<ACT>(b1[p.N + col]) : 0.0f;
      }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (row_lo + 32 * (i * Cfg::WM + wm) > row_last) break;   // block holds no rows
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = acc[i][0][4 * q + e] + bg[q][e], u = acc[i][1][4 * q + e] + bu[q][e];
          v[e] = silu_mul(g, u);
        }
        *reinterpret_cast<u32x2 *>(stg + row_in * 80 + (8 * q + 4 * khalf) * 2) =
            u32x2{pack2<ACT>(v[0], v[1]), pack2<ACT>(v[2], v[3])};
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rr = 16 * t + (lane >> 2), ch = lane & 3;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(stg + rr * 80 + ch * 16);
        const int r = row_lo + 32 * (i * Cfg::WM + wm) + rr;
        if (r <= row_last)
          __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(p.C + static_cast<size_t>(r) * p.N + n0 + 32 * wn + ch * 8));
      }
    }
    return;
  }
  float add[TN][4][4];    // bias (and int8 scale) per column of this lane
  float mul[TN][4][4];
  asm volatile("" ::: "memory");   // keep these loads out of the main loop's live range
  // Column c of this lane's 4-column run (j, q): wn WTN + 32 j + 8 q + 4 (lane / 32) + e.
  // One uniform choice per array, so each side is straight-line code.
  auto lcol = [&](int j, int q) { return wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf; };
  auto from_lds = [&](const char *base, int dt, float (&v)[TN][4][4]) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(base + lcol(j, q) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[j][q][e] = bits_to_f32_dyn(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))), dt);
      }
  };
  auto from_global = [&](const uint16_t *src, int dt, float (&v)[TN][4][4]) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][q][e] = bits_to_f32_dyn(src[n0 + lcol(j, q) + e], dt);
  };
  auto fill = [&](float x, float (&v)[TN][4][4]) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][q][e] = x;
  };
  if (bias_lds) from_lds(L.ep, p.bias_dt, add);
  else if (p.bias) from_global(p.bias, p.bias_dt, add);
  else fill(0.0f, add);
  if constexpr (kColScale) {
    if (cs_lds) from_lds(L.ep + kEpWaves * 256, ACT, mul);
    else from_global(p.S, ACT, mul);
  } else {
    fill(1.0f, mul);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (row_lo + 32 * (i * Cfg::WM + wm) > row_last) break;   // block holds no rows
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] * mul[j][q][e] + add[j][q][e];
        *reinterpret_cast<u32x2 *>(stg + row_in * 144 + (32 * j + 8 * q + 4 * khalf) * 2) =
            u32x2{pack2<ACT>(v[0], v[1]), pack2<ACT>(v[2], v[3])};
      }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rr = 8 * t + (lane >> 3), ch = lane & 7;
      const u32x4 val = *reinterpret_cast<const u32x4 *>(stg + rr * 144 + ch * 16);
      const int r = row_lo + 32 * (i * Cfg::WM + wm) + rr;
      if (r <= row_last)
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(p.C + static_cast<size_t>(r) * p.N + n0 + wn * Cfg::WTN + ch * 8));
    }
  }
}

}  // namespace qg
