// tile_gemm.hpp -- the matrix-core tile kernel behind the prefill GEMMs and
// the MoE grouped GEMMs (gfx950, v_mfma_f32_32x32x16_{bf16,f16}).
//
// One workgroup computes a BM x BN tile of C = A . W^T.  Per 64-wide step of
// K it stages A (raw 16-bit activations) and W (dequantized from the tiled
// integer codes by the workgroup itself) into LDS, double-buffered, and every
// wave reads its operand fragments from there with ds_read_b128.  Each packed
// weight is therefore dequantized once per workgroup and shared by all its
// waves -- the dequant-into-LDS structure that amortises the conversion over
// BM rows of activations.
//
// LDS rows are 128 bytes (64 k of 16-bit values) split into eight 16-byte
// chunks stored at chunk ^ (row % 8), so that the rows one fragment read
// touches spread over the banks (measured on gfx950: unswizzled rows run
// about 3x slower; this placement and chunk ^ ((row / 2) % 8) are within 1%).
//
// Dequant in this kernel: int4 w = fma(q, s, z - 8 s) rounded to nearest even.
// The fused multiply-add is exact before its one rounding, so this equals the
// once-rounded (q - 8) s + z whenever z - 8 s is exact in fp32.  It is when
// z = 0, and when |8 s| and |z| are within a factor 2^13 (fp16: 11
// significant bits each) or 2^16 (bf16: 8) of each other, so that their
// difference fits fp32's 24 bits; the dyadic test inputs always are.  A zero
// much smaller than 8 s (e.g. |z| < 2^-10 |s| in fp16) makes z - 8 s round,
// and the staged weight can then differ from the once-rounded value by one
// unit in the last place of the 16-bit type: within the GEMM tolerance, and
// not the bit-exact dequant contract, which qdequant_w4 implements directly.
// int8 per-channel stages the exact code q and multiplies the finished fp32
// sum by the channel's scale; int8 with group scales stages q * s rounded to
// nearest even.
#pragma once

#include "qg_common.hpp"

namespace qg {

enum TileMode { kDense = 0, kMoeFc1 = 1, kMoeFc2 = 2 };

// Tile of the MoE row space: rows [row0, row1) of the expert-sorted rows all
// belong to `expert`.
struct MoeTile {
  int expert, row0, row1, pad;
};

struct TileProblem {
  const uint16_t *A;         // dense: [M, K]; fc1: x [T, K] gathered; fc2: act [R, K]
  const uint8_t *B;          // tiled codes (expert 0 for MoE)
  const uint16_t *S, *Z;     // scales / zeros (expert 0 for MoE)
  const uint16_t *bias;      // dense: [N] or null; fc1: expert biases [E, 2N] or null
  uint16_t *C;               // dense: [M, N]; fc1: act [R, N]; fc2: y [R, N]
  int M, N, K;               // N = output columns (fc1: inter)
  int group;                 // 64 / 128 (w4); 0 (w8 per channel)
  int bias_dt;
  // MoE
  const int32_t *row_src;    // fc1: expert-sorted row -> token
  const MoeTile *tiles;      // tile list
  const int32_t *ntiles;     // number of valid entries in `tiles`
  size_t b_expert_stride;    // bytes of tiled codes per expert
  size_t s_expert_stride;    // scale/zero elements per expert
  int w_rows;                // rows of one expert's weight matrix
  int a_rows;                // rows of A (fc1: tokens; else M)
  // Dense split-K: K slices of kseg 64-k steps; a slice writes its fp32
  // partial tile to part + slice * M * N (no scale, bias or rounding) for a
  // separate reduction.  part == nullptr: one slice, finished output.
  float *part;
  int kseg;
};

// KG > 1: the workgroup runs KG groups of WM x WN waves on the same tile,
// group g on the g-th of KG consecutive parts of the K steps, each with its
// own LDS stages; at the end the groups' accumulators are added through LDS
// (group 0 first, then 1, ...) and group 0 writes the tile.  Twice the waves
// on half the steps each, for problems with too few tiles to fill the CUs.
template <int BM_, int BN_, int WM_, int WN_, int KG_ = 1>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, KG = KG_;
  static constexpr int BK = 64;
  static constexpr int NTG = 64 * WM * WN;             // threads of one K group
  static constexpr int NTHR = NTG * KG;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 subtiles per wave
  static constexpr int A_CHUNKS = BM * 8 / NTG;       // 16-byte A chunks per thread per step
  static constexpr int B_SLOTS = BN * 4 / NTG;        // 8-byte code runs per thread (w4)
  static constexpr int B_RUNS8 = BN * 8 / NTG;        // 8-byte code runs per thread (w8)
  static constexpr int STAGE = (BM + BN) * 128;       // bytes per LDS stage
  static constexpr int LDS = KG * 2 * STAGE;
  static_assert(A_CHUNKS >= 1 && B_SLOTS >= 1, "tile too small for the thread count");
  static_assert((KG - 1) * WM * WN * TM * TN * 16 * 64 * 4 <= LDS, "K-group partials fit the LDS");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// Dequantize one tiled int4 word (codes k0..k0+7, code e at its tiled nibble
// slot) with scale s and z8 = z - 8 s into 8 packed 16-bit values.
template <int ACT>
__device__ __forceinline__ u32x4 dequant_word_w4(uint32_t w, float s, float z8) {
  uint32_t m0 = w & 0x0F0F0F0Fu;          // nibble slots 0,2,4,6 -> codes 0,4,1,5
  uint32_t m1 = (w >> 4) & 0x0F0F0F0Fu;   // nibble slots 1,3,5,7 -> codes 2,6,3,7
  // Hide the masks' known zero bits from the optimizer: it would otherwise
  // turn each byte extraction into a 4-bit field extract plus a byte-0
  // convert instead of one v_cvt_f32_ubyteN.
  asm("" : "+v"(m0));
  asm("" : "+v"(m1));
  float q0 = static_cast<float>(m0 & 0xFFu), q4 = static_cast<float>((m0 >> 8) & 0xFFu);
  float q1 = static_cast<float>((m0 >> 16) & 0xFFu), q5 = static_cast<float>(m0 >> 24);
  float q2 = static_cast<float>(m1 & 0xFFu), q6 = static_cast<float>((m1 >> 8) & 0xFFu);
  float q3 = static_cast<float>((m1 >> 16) & 0xFFu), q7 = static_cast<float>(m1 >> 24);
  u32x4 r;
  r.x = pack2<ACT>(__builtin_fmaf(q0, s, z8), __builtin_fmaf(q1, s, z8));
  r.y = pack2<ACT>(__builtin_fmaf(q2, s, z8), __builtin_fmaf(q3, s, z8));
  r.z = pack2<ACT>(__builtin_fmaf(q4, s, z8), __builtin_fmaf(q5, s, z8));
  r.w = pack2<ACT>(__builtin_fmaf(q6, s, z8), __builtin_fmaf(q7, s, z8));
  return r;
}

// int8 codes with one scale per (channel, K-group): 8 offset-binary bytes ->
// 8 packed 16-bit values q * s, q = byte - 128.  (q - 128 folded into the
// fma: byte * s and 128 * s are exact in fp32 and so is their difference,
// which then rounds once, to nearest even, into the 16-bit type.)
template <int ACT>
__device__ __forceinline__ u32x4 dequant_run_w8(uint32_t lo, uint32_t hi, float s) {
  const float m = -128.0f * s;
  const uint32_t ws[2] = {lo, hi};
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float f0 = __builtin_fmaf(static_cast<float>(ws[h] & 0xFFu), s, m);
    const float f1 = __builtin_fmaf(static_cast<float>((ws[h] >> 8) & 0xFFu), s, m);
    const float f2 = __builtin_fmaf(static_cast<float>((ws[h] >> 16) & 0xFFu), s, m);
    const float f3 = __builtin_fmaf(static_cast<float>(ws[h] >> 24), s, m);
    r[2 * h] = pack2<ACT>(f0, f1);
    r[2 * h + 1] = pack2<ACT>(f2, f3);
  }
  return r;
}

// GS8 (int8 only): one scale per (channel, K-group of p.group), applied
// while dequantizing into LDS; otherwise int8 scales are per channel and
// multiply the finished sum.
template <class Cfg, int ACT, int WBITS, int MODE, bool GS8 = false>
__device__ __forceinline__ void tile_gemm(const TileProblem &p, int tile_m, int tile_n,
                                          char *lds, int slice = 0) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NTHR = Cfg::NTG;   // threads per K group
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  constexpr int GW = Cfg::WM * Cfg::WN;   // waves per K group
  const int lane = threadIdx.x & 63;
  const int kg = Cfg::KG > 1 ? static_cast<int>(threadIdx.x >> 6) / GW : 0;   // K group
  const int wave = (threadIdx.x >> 6) - kg * GW, tid = threadIdx.x - kg * NTHR;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int K = p.K;
  // This workgroup's 64-k steps: [sa, sb) (all of K unless split), and this K
  // group's part of them: [s0, s0 + nmine).  Every group runs `nsteps` loop
  // steps (the barriers are the workgroup's), the last group possibly a few
  // without matrix-core work when the steps do not divide evenly; those load
  // and stage a real step into the idle LDS stage.
  const int sa = p.part ? slice * p.kseg : 0;
  const int sb = p.part ? min(K / BK, sa + p.kseg) : K / BK;
  const int nsteps = (sb - sa + Cfg::KG - 1) / Cfg::KG;
  const int s0 = min(sa + kg * nsteps, sb - 1);
  const int nmine = max(0, min(nsteps, sb - sa - kg * nsteps));
  const int slast = s0 + max(nmine, 1) - 1;   // last real step of this group (a valid step)
  lds += kg * 2 * Cfg::STAGE;

  // ---- row sources for A -------------------------------------------------
  int row_lo, row_hi;         // valid global row range of this tile
  const uint8_t *Bbase = p.B;
  const uint16_t *Sbase = p.S, *Zbase = p.Z;
  [[maybe_unused]] const uint16_t *b1base = nullptr;   // fc1: this expert's [2 N] bias
  if constexpr (MODE == kDense) {
    row_lo = tile_m * BM;
    row_hi = min(p.M, row_lo + BM);
  } else {
    const MoeTile t = p.tiles[tile_m];
    row_lo = t.row0;
    row_hi = t.row1;
    Bbase += static_cast<size_t>(t.expert) * p.b_expert_stride;
    Sbase += static_cast<size_t>(t.expert) * p.s_expert_stride;
    if (Zbase) Zbase += static_cast<size_t>(t.expert) * p.s_expert_stride;
    if (MODE == kMoeFc1 && p.bias) b1base = p.bias + static_cast<size_t>(t.expert) * p.w_rows;
  }
  const int n0 = (MODE == kMoeFc1) ? tile_n * (BN / 2) : tile_n * BN;

  // A chunks owned by this thread: (row, chunk) pairs.  Rows past the tile's
  // end read the tile's first row and are masked to zero, so the loads stay
  // branch-free (a divergent branch around a load makes the wait-count
  // insertion fall back to draining every outstanding load, which would undo
  // the prefetch).
  const uint16_t *a_src[Cfg::A_CHUNKS];
  uint32_t a_keep[Cfg::A_CHUNKS];
  int a_lds[Cfg::A_CHUNKS];
#pragma unroll
  for (int c = 0; c < Cfg::A_CHUNKS; ++c) {
    const int idx = tid + c * NTHR;
    const int r = idx >> 3, ch = idx & 7;
    const int grow = row_lo + r;
    const bool live = grow < row_hi;
    a_lds[c] = swz(r, ch);
    a_keep[c] = live ? 0xFFFFFFFFu : 0u;
    const int srow = live ? grow : row_lo;
    size_t arow;
    if constexpr (MODE == kMoeFc1) arow = static_cast<size_t>(p.row_src[srow]);
    else arow = static_cast<size_t>(srow);
    a_src[c] = p.A + arow * K + ch * 8;
  }

  // B runs owned by this thread.
  // w4: slot = (16-row block bi, lane slot l); per step it reads the 8-byte
  //     half (words 2h, 2h+1) of the slot's 16 bytes, h = step % 2.
  // w8: run = (block bi, lane slot l, t): 8 bytes, one per step-block.
  constexpr int NB = (WBITS == 4) ? Cfg::B_SLOTS : Cfg::B_RUNS8;
  const uint8_t *b_src[NB];
  int b_lds0[NB], b_lds1[NB];
  size_t b_sidx[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int idx = tid + c * NTHR;
    int l, bi, t = 0;
    if constexpr (WBITS == 4) { l = idx & 63; bi = idx >> 6; }
    else { t = idx & 1; l = (idx >> 1) & 63; bi = idx >> 7; }
    const int nl = l & 15, j = l >> 4;
    const int lrow = bi * 16 + nl;                 // LDS row
    int wrow;                                      // weight row
    if constexpr (MODE == kMoeFc1)
      wrow = (lrow < BN / 2) ? n0 + lrow : p.N + n0 + (lrow - BN / 2);
    else
      wrow = n0 + lrow;
    if constexpr (WBITS == 4) {
      b_src[c] = Bbase + (static_cast<size_t>(wrow >> 4) * (K >> 7)) * 1024 + l * 16;
      b_lds0[c] = swz(lrow, j);        // word 2h   -> k-chunk j      (of the 64-k step)
      b_lds1[c] = swz(lrow, 4 + j);    // word 2h+1 -> k-chunk 4 + j
      b_sidx[c] = static_cast<size_t>(wrow) * (K / p.group);
    } else {
      b_src[c] = Bbase + (static_cast<size_t>(wrow >> 4) * (K >> 6)) * 1024 + l * 16 + t * 8;
      b_lds0[c] = swz(lrow, 4 * t + j);
      b_lds1[c] = 0;
      b_sidx[c] = GS8 ? static_cast<size_t>(wrow) * (K / p.group) : 0;
    }
  }

  // Register staging: two sets, so the global loads of step s + 2 are issued
  // while step s computes and step s + 1 waits in the other set -- two steps
  // of matrix-core work to hide the memory latency.
  struct Regs {
    u32x4 a[Cfg::A_CHUNKS];
    u32x2 b[NB];
    uint16_t s[NB], z[NB];
  };

  auto gload = [&](int step, Regs &r) {
    const int k0 = step * BK;
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c) r.a[c] = *reinterpret_cast<const u32x4 *>(a_src[c] + k0);
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if constexpr (WBITS == 4) {
        const int kb = step >> 1, h = step & 1;
        r.b[c] = *reinterpret_cast<const u32x2 *>(b_src[c] + static_cast<size_t>(kb) * 1024 + h * 8);
        const size_t gi = b_sidx[c] + (k0 / p.group);
        r.s[c] = Sbase[gi];
        r.z[c] = Zbase ? Zbase[gi] : uint16_t(0);   // no zeros: scale-only
      } else {
        r.b[c] = *reinterpret_cast<const u32x2 *>(b_src[c] + static_cast<size_t>(step) * 1024);
        if constexpr (GS8) r.s[c] = Sbase[b_sidx[c] + k0 / p.group];
      }
    }
  };

  auto lstore = [&](int stage, const Regs &r) {
    char *As = lds + stage * Cfg::STAGE;
    char *Bs = As + BM * 128;
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c) {
      const uint32_t k = a_keep[c];
      *reinterpret_cast<u32x4 *>(As + a_lds[c]) = u32x4{r.a[c].x & k, r.a[c].y & k, r.a[c].z & k, r.a[c].w & k};
    }
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if constexpr (WBITS == 4) {
        const float s = bits_to_f32<ACT>(r.s[c]);
        const float z8 = bits_to_f32<ACT>(r.z[c]) - 8.0f * s;
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) = dequant_word_w4<ACT>(r.b[c].x, s, z8);
        *reinterpret_cast<u32x4 *>(Bs + b_lds1[c]) = dequant_word_w4<ACT>(r.b[c].y, s, z8);
      } else if constexpr (GS8) {
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) =
            dequant_run_w8<ACT>(r.b[c].x, r.b[c].y, bits_to_f32<ACT>(r.s[c]));
      } else {
        *reinterpret_cast<u32x4 *>(Bs + b_lds0[c]) =
            (ACT == kFP16) ? w8_run_to_f16(r.b[c].x, r.b[c].y) : w8_run_to_bf16(r.b[c].x, r.b[c].y);
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jn = 0; jn < TN; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;

  // LDS rows this wave reads.
  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = wm * Cfg::WTM + 32 * i + (lane & 31);
#pragma unroll
  for (int jn = 0; jn < TN; ++jn) {
    if constexpr (MODE == kMoeFc1) {
      constexpr int HALF = TN / 2;
      const int base = (jn < HALF) ? wn * (Cfg::WTN / 2) + 32 * jn
                                   : BN / 2 + wn * (Cfg::WTN / 2) + 32 * (jn - HALF);
      b_row[jn] = base + (lane & 31);
    } else {
      b_row[jn] = wn * Cfg::WTN + 32 * jn + (lane & 31);
    }
  }
  const int khalf = lane >> 5;

  auto compute = [&](int stage) {
    const char *As = lds + stage * Cfg::STAGE;
    const char *Bs = As + BM * 128;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = 2 * ks + khalf;
      u32x4 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const u32x4 *>(As + swz(a_row[i], chunk));
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) bf[jn] = *reinterpret_cast<const u32x4 *>(Bs + swz(b_row[jn], chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) acc[i][jn] = mfma32x32x16<ACT>(af[i], bf[jn], acc[i][jn]);
    }
  };

  // One pipeline step: issue loads for step + 2 into `nxt2`, run the matrix
  // cores on LDS stage step % 2, then stage step + 1 (held in `nxt1`).  Both
  // are unconditional -- near the end they re-read the last step and store
  // into the idle LDS buffer, which is never read again -- because a load
  // inside a branch makes the wait-count insertion drain every outstanding
  // load before the store, which would cancel the prefetch.
  // Scheduling barriers keep that order: the compiler would otherwise hoist
  // the LDS stores (and the waits on their loads) above the matrix-core work
  // and sink the new loads below it.
  auto body = [&](int step, Regs &nxt1, Regs &nxt2) {   // step relative to s0
    gload(min(s0 + step + 2, slast), nxt2);
    __builtin_amdgcn_sched_barrier(0);
    if (Cfg::KG == 1 || step < nmine) compute(step & 1);
    __builtin_amdgcn_sched_barrier(0);
    lstore((step + 1) & 1, nxt1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };

  Regs r0, r1;
  gload(s0, r0);
  gload(min(s0 + 1, slast), r1);
  lstore(0, r0);
  __syncthreads();
  // Unrolled by two so the register sets are named statically: at an even
  // step r1 holds step + 1 and r0 receives step + 2; at an odd step the roles
  // swap.
  int step = 0;
  for (; step + 1 < nsteps; step += 2) {
    body(step, r1, r0);
    body(step + 1, r0, r1);
  }
  if (step < nsteps) body(step, r1, r0);

  if constexpr (Cfg::KG > 1) {
    // Add the K groups' accumulators: groups 1 .. KG - 1 leave theirs in LDS
    // (every stage is free: the last step ended with a barrier), group 0
    // adds them in group order and goes on to the epilogue.
    constexpr int PERW = TM * TN * 16 * 64;   // floats per wave
    float *red = reinterpret_cast<float *>(lds - kg * 2 * Cfg::STAGE);
    if (kg > 0) {
      float *dst = red + ((kg - 1) * GW + wave) * PERW;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
          for (int v = 0; v < 16; ++v) dst[((i * TN + jn) * 16 + v) * 64 + lane] = acc[i][jn][v];
    }
    __syncthreads();
    if (kg > 0) return;
    for (int g = 1; g < Cfg::KG; ++g) {
      const float *src = red + ((g - 1) * GW + wave) * PERW;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][jn][v] += src[((i * TN + jn) * 16 + v) * 64 + lane];
    }
  }

  // ---- epilogue -----------------------------------------------------------
  // 32x32 accumulator: value v of lane -> row 8*(v/4) + 4*(lane/32) + v%4,
  // column lane % 32.
  const int col_in = lane & 31;
  if constexpr (MODE == kDense) {
    if (p.part) {   // split-K slice: the raw fp32 partial sums
      float *dst = p.part + static_cast<size_t>(slice) * p.M * p.N;
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) {
        const int col = n0 + wn * Cfg::WTN + 32 * jn + col_in;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = row_lo + wm * Cfg::WTM + 32 * i + 8 * (v >> 2) + 4 * khalf + (v & 3);
            if (r < row_hi) dst[static_cast<size_t>(r) * p.N + col] = acc[i][jn][v];
          }
      }
      return;
    }
  }
  if constexpr (MODE == kMoeFc1) {
    constexpr int HALF = TN / 2;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jn = 0; jn < HALF; ++jn) {
        const int col = n0 + wn * (Cfg::WTN / 2) + 32 * jn + col_in;
        // fc1 biases of the gate and up rows (before the activation)
        const float bg = b1base ? bits_to_f32<ACT>(b1base[col]) : 0.0f;
        const float bu = b1base ? bits_to_f32<ACT>(b1base[p.N + col]) : 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = row_lo + wm * Cfg::WTM + 32 * i + 8 * (v >> 2) + 4 * khalf + (v & 3);
          if (r < row_hi) {
            const float g = acc[i][jn][v] + bg, u = acc[i][jn + HALF][v] + bu;
            const float a = silu_mul(g, u);
            p.C[static_cast<size_t>(r) * p.N + col] = f32_to_bits<ACT>(a);
          }
        }
      }
  } else {
#pragma unroll
    for (int jn = 0; jn < TN; ++jn) {
      const int col = n0 + wn * Cfg::WTN + 32 * jn + col_in;
      float cs = 1.0f, cb = 0.0f;
      if constexpr (WBITS == 8 && !GS8) cs = bits_to_f32<ACT>(Sbase[col]);
      if (MODE == kDense && p.bias) cb = bits_to_f32_dyn(p.bias[col], p.bias_dt);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = row_lo + wm * Cfg::WTM + 32 * i + 8 * (v >> 2) + 4 * khalf + (v & 3);
          if (r < row_hi) {
            float val = acc[i][jn][v];
            if constexpr (WBITS == 8 && !GS8) val *= cs;
            val += cb;
            p.C[static_cast<size_t>(r) * p.N + col] = f32_to_bits<ACT>(val);
          }
        }
    }
  }
}

}  // namespace qg
