// tile_dense.hpp -- the dense half of the dequantize-then-dense prefill path
// on gfx950: C = A . W^T with both operands 16-bit (bf16 or fp16) and
// K-contiguous, W being the weight matrix already dequantized into the
// caller's workspace.  vllm-omni cpu_int4.py, the int4 linear's dispatch
// (batches of at least dequant_threshold rows dequantize the whole weight
// and run one dense linear): here the same split, taken where the fused
// tiles would dequantize every weight once per row tile -- few output
// columns, many rows.
//
// Per 64-k step a workgroup moves its BM activation rows and BN weight rows
// (128 bytes each) from global memory straight into LDS (buffer_load ...
// lds, 16 bytes per lane, no VGPRs), NS - 1 steps ahead of use in NS stages,
// and runs v_mfma_f32_32x32x16 on them with fp32 accumulation.  Fragment
// addresses, the k order inside a step and the matrix instruction sequence
// are those of the fused direct-load tile (tile_big.hpp), so for the same W
// values every output is accumulated in the same order: without K slices
// or K groups the two paths give the same bits.
//
// LDS placement: a stage row is 128 bytes, its 16-byte chunk c stored at
// chunk c ^ ((row / 2) % 8); a direct load writes 64 consecutive 16-byte
// slots, so the swizzle is applied on the source side.  Rows past the end
// of A are read from the last valid row (a direct load cannot be masked);
// their outputs are never stored.  N is a multiple of BN.
#pragma once

#include <type_traits>

#include "qg_common.hpp"

namespace qg {

struct DenseProblem {
  const uint16_t *A;          // [M, K]
  const uint16_t *W;          // [N, K], dequantized
  const uint16_t *colscale;   // [N] (int8 per-channel scales, in A's type) or null
  const uint16_t *bias;       // [N] or null
  int bias_dt;
  uint16_t *C;                // [M, N]
  int M, N, K;
};

// NS LDS stages: the loads of step s + NS - 1 are issued at the top of step
// s, so a step's data has NS - 1 steps to arrive (the small tiles this path
// runs do little work per step, so one step ahead leaves the memory latency
// exposed).
template <int BM_, int BN_, int WM_, int WN_, int NS_>
struct DenseCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int NTHR = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 accumulators per wave
  static constexpr int A_DMA = BM * 8 / NTHR;          // 16-byte direct loads per thread per step
  static constexpr int B_DMA = BN * 8 / NTHR;
  static constexpr int STAGE_A = BM * 128, STAGE_B = BN * 128;
  static_assert(NTHR == 512, "eight waves");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && A_DMA >= 1 && B_DMA >= 1, "tile shape");
  static_assert(NS >= 2 && NS <= 4 && NS * (STAGE_A + STAGE_B) <= 160 * 1024, "LDS stages");
  static_assert((NS - 2) * (A_DMA + B_DMA) < 64, "vmcnt field");
};

// The stages are separate LDS objects (with one array and a stage index the
// compiler's wait-count pass cannot tell a stage being read from one being
// loaded, and waits for every direct load before each step's first read).
struct DenseLds {
  char *a[4];
  char *b[4];
};

// s_waitcnt with vmcnt(n), lgkmcnt(0), expcnt untouched.
constexpr int dense_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

template <class Cfg, int ACT>
__device__ __forceinline__ void dense_tile_gemm(const DenseProblem &p, int tm, int tn,
                                                const DenseLds &L) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, NS = Cfg::NS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int K = p.K, nsteps = K / 64;
  const int row_lo = tm * Cfg::BM, row_last = min(p.M, row_lo + Cfg::BM) - 1;
  const int col_lo = tn * Cfg::BN;

  constexpr int kRsrcFlags = 0x00020000;
  const uint32_t kb = static_cast<uint32_t>(K) * 2u;   // bytes per row
  const auto rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.A), 0,
                                                    static_cast<int>(static_cast<uint32_t>(p.M) * kb), kRsrcFlags);
  const auto rB = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.W), 0,
                                                    static_cast<int>(static_cast<uint32_t>(p.N) * kb), kRsrcFlags);

  // Slot q = (wave * X_DMA + i) * 64 + lane of a stage is row q / 8, placed
  // chunk q % 8, holding the row's chunk (q % 8) ^ ((row / 2) % 8).
  uint32_t a_voff[Cfg::A_DMA], b_voff[Cfg::B_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::A_DMA; ++i) {
    const int q = (wave * Cfg::A_DMA + i) * 64 + lane;
    const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    a_voff[i] = static_cast<uint32_t>(min(row_lo + r, row_last)) * kb + c * 16;
  }
#pragma unroll
  for (int i = 0; i < Cfg::B_DMA; ++i) {
    const int q = (wave * Cfg::B_DMA + i) * 64 + lane;
    const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    b_voff[i] = static_cast<uint32_t>(col_lo + r) * kb + c * 16;
  }
  // Step `step` into stage ST; past the last step the last one is loaded
  // again (into a stage no later step reads), so every step issues the same
  // number of loads and one wait count fits all.
  auto issue = [&](auto STc, int step) {
    constexpr int ST = decltype(STc)::value;
    const int sk = min(step, nsteps - 1) * 128;
    char *da = L.a[ST] + wave * Cfg::A_DMA * 1024;
    char *db = L.b[ST] + wave * Cfg::B_DMA * 1024;
#pragma unroll
    for (int i = 0; i < Cfg::A_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rA, (__attribute__((address_space(3))) void *)(da + i * 1024), 16, a_voff[i], sk, 0, 0);
#pragma unroll
    for (int i = 0; i < Cfg::B_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rB, (__attribute__((address_space(3))) void *)(db + i * 1024), 16, b_voff[i], sk, 0, 0);
  };

  // Fragments: sub-step ks covers k 16 ks .. 16 ks + 15 of the step; lane
  // reads row (wave tile row + 32 i + lane % 32), chunk 2 ks + lane / 32,
  // placed at that ^ ((lane / 2) % 8).
  const int khalf = lane >> 5;
  const int g = khalf ^ ((lane >> 1) & 7);
  int a_addr[4], b_addr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    a_addr[ks] = (wm * Cfg::WTM + (lane & 31)) * 128 + (((2 * ks) ^ g) << 4);
    b_addr[ks] = (wn * Cfg::WTN + (lane & 31)) * 128 + (((2 * ks) ^ g) << 4);
  }
  struct Frags {
    u32x4 a[TM], b[TN];
  };
  auto fread = [&](const char *As, const char *Bs, int ks, Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const u32x4 *>(As + a_addr[ks] + 4096 * i);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const u32x4 *>(Bs + b_addr[ks] + 4096 * j);
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
  auto mma = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<ACT>(f.b[j], f.a[i], acc[i][j]);
  };
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // After a step's issue, the loads of the next step are the oldest but
  // those of the NS - 2 steps after it.
  constexpr int WAIT_NEXT = dense_wait((NS - 2) * (Cfg::A_DMA + Cfg::B_DMA));

  // Step s on stage I = s % NS: issue step s + NS - 1 into stage
  // (s - 1) % NS (last read in step s - 1, before the barrier that ended
  // it), run the four sub-steps, wait for this wave's loads of step s + 1,
  // meet the other waves.
  auto body = [&](auto Ic, int step) {
    constexpr int I = decltype(Ic)::value;
    issue(std::integral_constant<int, (I + NS - 1) % NS>{}, step + NS - 1);
    __builtin_amdgcn_sched_barrier(0);
    const char *As = L.a[I], *Bs = L.b[I];
    Frags f0, f1;
    fread(As, Bs, 0, f0);
    fread(As, Bs, 1, f1);
    mma(f0);
    fread(As, Bs, 2, f0);
    mma(f1);
    fread(As, Bs, 3, f1);
    mma(f0);
    mma(f1);
    // Fragment reads one sub-step ahead of the matrix instructions.
    constexpr int NR = TM + TN, NM = TM * TN;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
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
  // The re-issued loads of the last steps are still in flight: let them land
  // before the workgroup (and its LDS) ends.
  __builtin_amdgcn_s_waitcnt(dense_wait(0));

  // Epilogue: value v of acc[i][j] is C[row][col], row = wave tile row +
  // 32 i + lane % 32, col = wave tile column + 32 j + 8 (v / 4) +
  // 4 (lane / 32) + v % 4; C = RNE(acc * channel scale + bias), the fused
  // tiles' expression.
  float add[TN][4][4], mul[TN][4][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = col_lo + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf + e;
        add[j][q][e] = p.bias ? bits_to_f32_dyn(p.bias[col], p.bias_dt) : 0.0f;
        mul[j][q][e] = p.colscale ? bits_to_f32<ACT>(p.colscale[col]) : 1.0f;
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
