// tile_w8dir.hpp -- W8A16 on gfx950 (one scale per output channel, or per
// channel and 64- or 128-k group): the
// int8 weight codes go from their tiled layout straight into LDS (buffer_load
// ... lds, one 1 KiB block of 16 rows x 64 k per load instruction, no VGPRs),
// and each wave turns the code fragments it reads into exact 16-bit operands
// in registers (the codes are small integers, so nothing is rounded); a
// channel scale is applied to the finished sum, a group scale during the
// conversion (q s rounded once, as the fused tiles do: a lane's 8 codes lie
// in one group, so one scale per row and step, loaded with the step's
// direct loads into a register ring).  Against the fused tiles,
// which convert every code once per workgroup and stage the 16-bit weights
// in LDS, the weight bytes in LDS halve and the conversion's LDS writes go
// away, at the price of converting each code once per wave row.  A tile can
// also cover one K slice and store its unscaled fp32 sums as partials for
// the split-K reduction.
//
// Per 64-k step a workgroup moves its BM activation rows (128 bytes each)
// and its BN / 16 code blocks into one of NS LDS stages, NS - 1 steps ahead;
// each stage a separate LDS object (with one array and a stage index the
// compiler's wait-count pass cannot tell a stage being read from one being
// loaded).  Fragment addresses, the k order inside a step and the matrix
// instruction sequence are those of the fused direct-load tile, so for the
// same codes every output is accumulated in the same order and the two give
// the same bits.
//
// LDS placement: activations as in the fused tile (16-byte chunk c of row r
// at chunk c ^ ((r / 2) % 8)).  Code block b (rows 16 b .. 16 b + 15) at byte
// 1024 b, as stored: slot (j, nl) holds row nl, k-chunk j (k 8 j .. 8 j + 7)
// in its first 8 bytes and chunk 4 + j in its last 8.  A lane reads its
// whole slot, once for sub-steps ks and ks + 2 (k-chunks 2 ks + lane / 32 and
// that + 4), so 16 lanes read 256 contiguous bytes.
#pragma once

#include <type_traits>

#include "qg_common.hpp"
#include "tile_gemm.hpp"

namespace qg {

struct W8DirProblem {
  const uint16_t *A;          // [M, K]
  const uint8_t *B;           // tiled int8 codes (offset binary), [N, K]
  const uint16_t *S;          // [N] channel scales or [N, K / group] group scales, A's type
  const uint16_t *bias;       // [N] or null
  int bias_dt;
  uint16_t *C;                // [M, N]
  int M, N, K;
  int group;                  // 64 or 128 (group scales), 0 (channel scales)
  float *part;                // K slices: fp32 partials [nsplit][M][N], else null
  int kseg;                   // K slices: 64-k steps per slice
};

template <int BM_, int BN_, int WM_, int WN_, int NS_>
struct W8DirCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int NTHR = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 accumulators per wave
  static constexpr int A_DMA = BM * 8 / NTHR;          // 16-byte direct loads per thread per step
  static constexpr int B_BLK = BN / 16;                // code blocks per step
  static constexpr int B_DMA = B_BLK * 64 / NTHR;      // block loads per thread per step
  static constexpr int BLK_PITCH = 1024;
  static constexpr int STAGE_A = BM * 128, STAGE_B = B_BLK * BLK_PITCH;
  static_assert(NTHR == 512, "eight waves");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && A_DMA >= 1 && B_DMA >= 1, "tile shape");
  static_assert(NS >= 2 && NS <= 4 && NS * (STAGE_A + STAGE_B) <= 160 * 1024, "LDS stages");
  static_assert((NS - 2) * (A_DMA + B_DMA + TN) < 64, "vmcnt field");
};

struct W8DirLds {
  char *a[4];
  char *b[4];
};

// s_waitcnt with vmcnt(n), lgkmcnt(0), expcnt untouched.
constexpr int w8dir_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// SPLIT: the tile covers 64-k steps slice * kseg .. + kseg - 1 (fewer in the
// last slice) and stores its unscaled fp32 sums as that slice's partials.
template <class Cfg, int ACT, bool GS, bool SPLIT = false>
__device__ __forceinline__ void w8dir_tile_gemm(const W8DirProblem &p, int tm, int tn,
                                                const W8DirLds &L, int slice = 0) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, NS = Cfg::NS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int K = p.K;
  const int k0 = SPLIT ? slice * p.kseg : 0;                        // first step
  const int nsteps = SPLIT ? min(K / 64 - k0, p.kseg) : K / 64;     // steps walked
  const int row_lo = tm * Cfg::BM, row_last = min(p.M, row_lo + Cfg::BM) - 1;
  const int col_lo = tn * Cfg::BN;

  constexpr int kRsrcFlags = 0x00020000;
  const uint32_t kb = static_cast<uint32_t>(K) * 2u;   // activation bytes per row
  const auto rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.A), 0,
                                                    static_cast<int>(static_cast<uint32_t>(p.M) * kb), kRsrcFlags);
  const auto rB = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.B), 0,
                                                    static_cast<int>(static_cast<uint32_t>(p.N) * static_cast<uint32_t>(K)),
                                                    kRsrcFlags);

  // A: slot q = (wave * A_DMA + i) * 64 + lane of a stage is row q / 8,
  // placed chunk q % 8, holding the row's chunk (q % 8) ^ ((row / 2) % 8).
  uint32_t a_voff[Cfg::A_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::A_DMA; ++i) {
    const int q = (wave * Cfg::A_DMA + i) * 64 + lane;
    const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    a_voff[i] = static_cast<uint32_t>(min(row_lo + r, row_last)) * kb + c * 16;
  }
  // B: load i of a wave brings block (wave * B_DMA + i): the 1 KiB of codes
  // of rows col_lo + 16 blk .. + 15 at the step's 64 k, lane l its slot l.
  uint32_t b_voff[Cfg::B_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::B_DMA; ++i) {
    const int blk = wave * Cfg::B_DMA + i;
    b_voff[i] = static_cast<uint32_t>(col_lo / 16 + blk) * static_cast<uint32_t>(K / 64) * 1024u + lane * 16;
  }
  // Group scales: stage ST's scale of row block j of this lane's rows.
  [[maybe_unused]] uint16_t sreg[NS][TN];
  [[maybe_unused]] const int kg = GS ? K / p.group : 1;
  // Step `step` into stage ST; past the last step the last one is loaded
  // again (into a stage no later step reads), so every step issues the same
  // number of loads and one wait count fits all.
  auto issue = [&](auto STc, int step) {
    constexpr int ST = decltype(STc)::value;
    const int s = k0 + min(step, nsteps - 1);
    char *da = L.a[ST] + wave * Cfg::A_DMA * 1024;
#pragma unroll
    for (int i = 0; i < Cfg::A_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rA, (__attribute__((address_space(3))) void *)(da + i * 1024), 16, a_voff[i], s * 128, 0, 0);
#pragma unroll
    for (int i = 0; i < Cfg::B_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rB, (__attribute__((address_space(3))) void *)(L.b[ST] + (wave * Cfg::B_DMA + i) * Cfg::BLK_PITCH),
          16, b_voff[i], s * 1024, 0, 0);
    if constexpr (GS) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = col_lo + wn * Cfg::WTN + 32 * j + (lane & 31);
        sreg[ST][j] = p.S[static_cast<size_t>(n) * kg + (s * 64) / p.group];
      }
    }
  };

  // Fragments: sub-step ks covers k 16 ks .. 16 ks + 15 of the step; lane
  // takes k-chunk c = 2 ks + lane / 32 of its row (lane % 32 within the
  // 32-row block).  Activations: chunk c at c ^ ((row / 2) % 8).  Codes:
  // row n of the tile in block n / 16, slot (c % 4) 16 + n % 16; for
  // kp = 0, 1 the slot of chunk 2 kp + lane / 32 also holds chunk
  // 2 (kp + 2) + lane / 32.
  const int khalf = lane >> 5;
  const int g = khalf ^ ((lane >> 1) & 7);
  int a_addr[4], b_addr[2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) a_addr[ks] = (wm * Cfg::WTM + (lane & 31)) * 128 + (((2 * ks) ^ g) << 4);
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    const int n = wn * Cfg::WTN + (lane & 31);
    b_addr[kp] = (n >> 4) * Cfg::BLK_PITCH + (16 * (2 * kp + khalf) + (n & 15)) * 16;
  }
  auto read_a = [&](const char *As, int ks, u32x4 (&a)[TM]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const u32x4 *>(As + a_addr[ks] + 4096 * i);
  };
  auto read_b = [&](const char *Bs, int kp, u32x4 (&b)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j)   // 32 rows further: two blocks further
      b[j] = *reinterpret_cast<const u32x4 *>(Bs + b_addr[kp] + 2 * Cfg::BLK_PITCH * j);
  };

  // Weights as the row operand, activations as the column operand: acc[i][j]
  // holds C^T, a lane one row of C (32 i + lane % 32) and 16 of its columns,
  // four consecutive ones per group of four values.
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // Sub-step on activation fragments a and the code slots b: the slots'
  // first (HI = 0) or last 8 bytes.
  auto mma = [&](auto HIc, auto STc, const u32x4 (&a)[TM], const u32x4 (&b)[TN]) {
    constexpr int HI = decltype(HIc)::value, ST = decltype(STc)::value;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint32_t lo = b[j][2 * HI], hi = b[j][2 * HI + 1];
      u32x4 w;
      if constexpr (GS) w = dequant_run_w8<ACT>(lo, hi, bits_to_f32<ACT>(sreg[ST][j]));
      else w = (ACT == kFP16) ? w8_run_to_f16(lo, hi) : w8_run_to_bf16(lo, hi);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][j] = mfma32x32x16<ACT>(w, a[i], acc[i][j]);
    }
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // After a step's issue, the loads of the next step are the oldest but
  // those of the NS - 2 steps after it.
  constexpr int WAIT_NEXT = w8dir_wait((NS - 2) * (Cfg::A_DMA + Cfg::B_DMA + (GS ? TN : 0)));

  // Step s on stage I = s % NS: issue step s + NS - 1 into stage
  // (s - 1) % NS (last read in step s - 1, before the barrier that ended
  // it), run the four sub-steps, wait for this wave's loads of step s + 1,
  // meet the other waves.
  auto body = [&](auto Ic, int step) {
    constexpr int I = decltype(Ic)::value;
    issue(std::integral_constant<int, (I + NS - 1) % NS>{}, step + NS - 1);
    __builtin_amdgcn_sched_barrier(0);
    const char *As = L.a[I], *Bs = L.b[I];
    u32x4 a0[TM], a1[TM], b0[TN], b1[TN];
    read_a(As, 0, a0);
    read_b(Bs, 0, b0);
    read_a(As, 1, a1);
    read_b(Bs, 1, b1);
    mma(H0{}, Ic, a0, b0);   // ks 0
    read_a(As, 2, a0);
    mma(H0{}, Ic, a1, b1);   // ks 1
    read_a(As, 3, a1);
    mma(H1{}, Ic, a0, b0);   // ks 2
    mma(H1{}, Ic, a1, b1);   // ks 3
    // Fragment reads one sub-step ahead of the matrix instructions.
    constexpr int NM = TM * TN;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + TN), 0);   // reads: ks 0, 1 (codes for all four)
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);              // MFMA ks 0
    __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);              // reads ks 2
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);              // MFMA ks 1
    __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);              // reads ks 3
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);              // MFMA ks 2
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);              // MFMA ks 3
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    barrier();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  // Prologue: steps 0 .. NS - 2 into stages 0 .. NS - 2, then wait for step 0.
  issue(S0{}, 0);
  if constexpr (NS > 2) issue(S1{}, 1);
  if constexpr (NS > 3) issue(S2{}, 2);
  __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
  barrier();
  int step = 0;
  for (; step + NS <= nsteps; step += NS) {
    body(S0{}, step);
    body(S1{}, step + 1);
    if constexpr (NS > 2) body(S2{}, step + 2);
    if constexpr (NS > 3) body(S3{}, step + 3);
  }
  if (step < nsteps) body(S0{}, step);
  if (step + 1 < nsteps) body(S1{}, step + 1);
  if constexpr (NS > 2)
    if (step + 2 < nsteps) body(S2{}, step + 2);
  // The re-issued loads of the last steps land before the workgroup (and its
  // LDS) ends.
  __builtin_amdgcn_s_waitcnt(w8dir_wait(0));

  // Epilogue: value v of acc[i][j] is C[row][col], row = wave tile row +
  // 32 i + lane % 32, col = wave tile column + 32 j + 8 (v / 4) +
  // 4 (lane / 32) + v % 4; C = RNE(acc * channel scale + bias), the fused
  // tiles' expression.  K slices: the sums as they are, 16 bytes a store.
  if constexpr (SPLIT) {
    float *P = p.part + static_cast<size_t>(slice) * p.M * p.N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = row_lo + wm * Cfg::WTM + 32 * i + (lane & 31);
      if (r > row_last) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = col_lo + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf;
          *reinterpret_cast<f32x4 *>(P + static_cast<size_t>(r) * p.N + col) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
    }
    return;
  }
  float add[TN][4][4], mul[TN][4][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = col_lo + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf + e;
        add[j][q][e] = p.bias ? bits_to_f32_dyn(p.bias[col], p.bias_dt) : 0.0f;
        mul[j][q][e] = GS ? 1.0f : bits_to_f32<ACT>(p.S[col]);
      }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = row_lo + wm * Cfg::WTM + 32 * i + (lane & 31);
    if (r > row_last) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = col_lo + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] * mul[j][q][e] + add[j][q][e];
        *reinterpret_cast<u32x2 *>(p.C + static_cast<size_t>(r) * p.N + col) =
            u32x2{pack2<ACT>(v[0], v[1]), pack2<ACT>(v[2], v[3])};
      }
  }
}

}  // namespace qg
