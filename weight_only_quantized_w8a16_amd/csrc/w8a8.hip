// w8a8.hip -- int8 x int8 GEMM with tensor, token and channel scales (W8A8,
// SmoothQuant) on gfx950:
//
//   C[m, n] = RNE_out( float(sum_k A[m, k] * B[n, k]) * alpha_row[m] * alpha_col[n] )
//
// alpha_row is one value (per tensor) or one per activation row (per token),
// alpha_col one value or one per output channel.  Sources: "acext User Guide
// (v1.7)", 1.2.2 w8a8 GEMM (the runner's arguments: A, B, quant mode, column
// and row scales, C, m, n, k, workspace, stream; the output type is the
// template parameter) and 1.3.4 SmoothQuant (both operands stay integer; four
// variants: activations per tensor or per token, weights per tensor or per
// channel).
//
// Both operands are K-contiguous int8 rows, which is the operand order of the
// int8 matrix instruction, so nothing is repacked: a workgroup moves 128-k
// slabs of its BM activation rows and BN weight rows from global memory
// straight into LDS (buffer_load ... lds, 16 bytes per lane, no VGPRs), one
// step ahead of use in two stages, and runs v_mfma_i32_32x32x32_i8 on them.
// The int32 accumulators are exact (|sum| <= 2^14 k < 2^31 for the k the
// host accepts); the scales are applied once, in fp32, in the epilogue.
//
// LDS placement (as in the weight-only tiles): a stage row is 128 bytes, its
// 16-byte chunk c stored at chunk c ^ ((row / 2) % 8), so the 16 rows a lane
// group reads at one chunk land in 16 distinct bank groups.  A direct load
// writes 64 consecutive 16-byte slots, so the swizzle is applied on the
// source side.  Rows past the end of A or B are read from the last valid row
// (a direct load cannot be masked); their outputs are never stored.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "qg_common.hpp"
#include "qg_launch.hpp"

namespace qg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

struct W8A8Problem {
  const int8_t *A;       // [M, K]
  const int8_t *B;       // [N, K]
  const float *arow;     // [M] (per token) or [1]
  const float *acol;     // [N] (per channel) or [1]
  void *C;               // [M, N], out dtype
  int32_t *part;         // split-K: int32 partial sums [nsplit, M, N]; else null
  int M, N, K;
  int per_token, per_channel;
  int kseg;              // 128-k steps per K slice (split-K)
};

// NS LDS stages, loads issued NS - 1 steps ahead.
template <int BM_, int BN_, int WM_, int WN_, int NS_ = 2>
struct W8Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int NTHR = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 accumulators per wave
  static constexpr int A_DMA = BM * 8 / NTHR;          // 16-byte direct loads per thread per step
  static constexpr int B_DMA = BN * 8 / NTHR;
  static_assert(NTHR == 512, "eight waves");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && A_DMA >= 1 && B_DMA >= 1, "tile shape");
  static_assert(NS >= 2 && NS <= 4 && NS * (BM + BN) * 128 <= 160 * 1024, "LDS stages");
};

// Output element conversion.
template <int OUT>
__device__ __forceinline__ void store4(void *C, size_t off, const float (&v)[4]) {
  if constexpr (OUT == QG_FP32) {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(C) + off) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(C) + off) =
        u32x2{pack2<OUT>(v[0], v[1]), pack2<OUT>(v[2], v[3])};
  }
}

// Workgroup b runs on XCD b % 8.  Each XCD takes a contiguous run of the
// tile order, so neighbouring tiles share an L2.
__device__ __forceinline__ int w8a8_linear_id() {
  const int bid = blockIdx.x, nblk = gridDim.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
}

// Tile order: bands of four row tiles walked column by column, so one weight
// tile serves the band's row tiles while it is in L2.
__device__ __forceinline__ void w8a8_tile(int id, int tiles_m, int tiles_n, int &tm, int &tn) {
  constexpr int G = 4;
  const int band = id / (G * tiles_n);
  const int first = band * G, gsz = min(G, tiles_m - first);
  const int in = id - band * G * tiles_n;
  tm = first + in % gsz;
  tn = in / gsz;
}

// The two LDS stages of each operand are separate objects: with one array
// and a stage index the compiler's wait-count pass cannot tell the stage
// being read from the one being loaded, and made every step wait for the
// next step's direct loads before its first fragment read.
struct W8Lds {
  char *a[4];
  char *b[4];
};

template <class Cfg, int OUT, bool SPLIT>
__device__ __forceinline__ void w8a8_tile_gemm(const W8A8Problem &p, int tiles_m, int tiles_n,
                                               const W8Lds &L) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int K = p.K, nsteps = K / 128;

  const int id = w8a8_linear_id();
  const int per = tiles_m * tiles_n;
  const int slice = SPLIT ? id / per : 0;
  int tm, tn;
  w8a8_tile(id - slice * per, tiles_m, tiles_n, tm, tn);
  const int s0 = SPLIT ? slice * p.kseg : 0;
  const int s1 = SPLIT ? min(nsteps, s0 + p.kseg) : nsteps;
  const int row_lo = tm * Cfg::BM, row_last = min(p.M, row_lo + Cfg::BM) - 1;
  const int col_lo = tn * Cfg::BN, col_last = min(p.N, col_lo + Cfg::BN) - 1;

  constexpr int kRsrcFlags = 0x00020000;
  const auto rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.A), 0,
                                                    static_cast<int>(static_cast<uint32_t>(p.M) * static_cast<uint32_t>(K)), kRsrcFlags);
  const auto rB = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.B), 0,
                                                    static_cast<int>(static_cast<uint32_t>(p.N) * static_cast<uint32_t>(K)), kRsrcFlags);

  // Slot q = (wave * X_DMA + i) * 64 + lane of a stage is row q / 8, placed
  // chunk q % 8, holding the row's chunk (q % 8) ^ ((row / 2) % 8).
  uint32_t a_voff[Cfg::A_DMA], b_voff[Cfg::B_DMA];
#pragma unroll
  for (int i = 0; i < Cfg::A_DMA; ++i) {
    const int q = (wave * Cfg::A_DMA + i) * 64 + lane;
    const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    a_voff[i] = static_cast<uint32_t>(min(row_lo + r, row_last)) * static_cast<uint32_t>(K) + c * 16;
  }
#pragma unroll
  for (int i = 0; i < Cfg::B_DMA; ++i) {
    const int q = (wave * Cfg::B_DMA + i) * 64 + lane;
    const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
    b_voff[i] = static_cast<uint32_t>(min(col_lo + r, col_last)) * static_cast<uint32_t>(K) + c * 16;
  }
  // Step `step` into stage ST; past the slice's last step its last step is
  // loaded again (into a stage no later step reads), so every step issues
  // the same number of loads and one wait count fits all.
  auto issue = [&](auto STc, int step) {
    constexpr int ST = decltype(STc)::value;
    const int sk = min(step, s1 - 1) * 128;
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

  // Fragments: sub-step ks covers k bytes 32 ks .. 32 ks + 31; lane reads
  // row (wave tile row + 32 i + lane % 32), chunk 2 ks + lane / 32, placed at
  // that ^ ((lane / 2) % 8) (32 i and the wave tile leave (row / 2) % 8
  // unchanged).  The two operands read the same k bytes per lane, so the
  // instruction's k order within a fragment does not matter.
  const int khalf = lane >> 5;
  const int g = khalf ^ ((lane >> 1) & 7);
  int a_addr[4], b_addr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    a_addr[ks] = (wm * Cfg::WTM + (lane & 31)) * 128 + (((2 * ks) ^ g) << 4);
    b_addr[ks] = (wn * Cfg::WTN + (lane & 31)) * 128 + (((2 * ks) ^ g) << 4);
  }
  struct Frags {
    i32x4 a[TM], b[TN];
  };
  auto fread = [&](const char *As, const char *Bs, int ks, Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const i32x4 *>(As + a_addr[ks] + 4096 * i);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const i32x4 *>(Bs + b_addr[ks] + 4096 * j);
  };

  // Weights as the row operand, activations as the column operand: acc[i][j]
  // holds C^T, a lane one row of C (32 i + lane % 32) and 16 of its columns,
  // four consecutive ones per group of four values.
  i32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
  auto mma = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  constexpr int NS = Cfg::NS;
  // vmcnt: after a step's issue the next step's loads are the oldest but
  // those of the NS - 2 steps after it; lgkmcnt(0).
  constexpr int NWAIT = (NS - 2) * (Cfg::A_DMA + Cfg::B_DMA);
  constexpr int WAIT_NEXT = (NWAIT & 15) | ((NWAIT >> 4) << 14) | (7 << 4);

  // Step s on stage I = (s - s0) % NS: issue step s + NS - 1 into stage
  // (I - 1) % NS (last read in step s - 1, before the barrier that ended it),
  // run the four sub-steps, wait for this wave's loads of step s + 1, meet
  // the other waves.
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

  issue(S0{}, s0);
  if constexpr (NS > 2) issue(S1{}, s0 + 1);
  if constexpr (NS > 3) issue(S2{}, s0 + 2);
  __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
  barrier();
  int step = s0;
  for (; step + NS <= s1; step += NS) {
    body(S0{}, step);
    body(S1{}, step + 1);
    if constexpr (NS > 2) body(S2{}, step + 2);
    if constexpr (NS > 3) body(S3{}, step + 3);
  }
  if (step < s1) body(S0{}, step);
  if (step + 1 < s1) body(S1{}, step + 1);
  if constexpr (NS > 2)
    if (step + 2 < s1) body(S2{}, step + 2);
  // The re-issued loads of the last steps land before the workgroup (and its
  // LDS) ends.
  __builtin_amdgcn_s_waitcnt(7 << 4);

  // Epilogue: value v of acc[i][j] is C[row][col], row = wave tile row +
  // 32 i + lane % 32, col = wave tile column + 32 j + 8 (v / 4) +
  // 4 (lane / 32) + v % 4.  The column scales of this lane's 16 columns are
  // read once (clamped to the last column; columns past it are not stored).
  [[maybe_unused]] float cs[TN][4][4];
  if constexpr (!SPLIT) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = min(col_lo + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf + e, col_last);
          cs[j][q][e] = p.acol[p.per_channel ? col : 0];
        }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = row_lo + wm * Cfg::WTM + 32 * i + (lane & 31);
    if (r > row_last) continue;
    if constexpr (SPLIT) {
      int32_t *dst = p.part + static_cast<size_t>(slice) * p.M * p.N + static_cast<size_t>(r) * p.N;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = col_lo + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf;
          if (col <= col_last)
            *reinterpret_cast<i32x4 *>(dst + col) =
                i32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
    } else {
      const float ar = p.arow[p.per_token ? r : 0];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = col_lo + wn * Cfg::WTN + 32 * j + 8 * q + 4 * khalf;
          if (col > col_last) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(acc[i][j][4 * q + e]) * ar * cs[j][q][e];
          store4<OUT>(p.C, static_cast<size_t>(r) * p.N + col, v);
        }
    }
  }
}

template <class Cfg, int OUT, bool SPLIT>
__global__ __launch_bounds__(Cfg::NTHR) void k_w8a8(W8A8Problem p, int tiles_m, int tiles_n) {
  constexpr int SA = Cfg::BM * 128, SB = Cfg::BN * 128;
  __shared__ __attribute__((aligned(16))) char a0[SA];
  __shared__ __attribute__((aligned(16))) char a1[SA];
  __shared__ __attribute__((aligned(16))) char a2[Cfg::NS > 2 ? SA : 16];
  __shared__ __attribute__((aligned(16))) char a3[Cfg::NS > 3 ? SA : 16];
  __shared__ __attribute__((aligned(16))) char b0[SB];
  __shared__ __attribute__((aligned(16))) char b1[SB];
  __shared__ __attribute__((aligned(16))) char b2[Cfg::NS > 2 ? SB : 16];
  __shared__ __attribute__((aligned(16))) char b3[Cfg::NS > 3 ? SB : 16];
  w8a8_tile_gemm<Cfg, OUT, SPLIT>(p, tiles_m, tiles_n, W8Lds{{a0, a1, a2, a3}, {b0, b1, b2, b3}});
}

// Split-K: C = RNE_out(float(sum of the slices' int32 partials) * scales);
// the integer sum is exact, so the slice order does not matter.
template <int OUT>
__global__ __launch_bounds__(256) void k_w8a8_reduce(W8A8Problem p, int nsplit) {
  const long long q = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t mn = static_cast<size_t>(p.M) * p.N;
  if (q >= static_cast<long long>(mn / 4)) return;
  i32x4 s = *reinterpret_cast<const i32x4 *>(p.part + 4 * q);
  for (int sl = 1; sl < nsplit; ++sl) s += *reinterpret_cast<const i32x4 *>(p.part + sl * mn + 4 * q);
  const int r = static_cast<int>((4 * q) / p.N), col = static_cast<int>((4 * q) % p.N);
  const float ar = p.arow[p.per_token ? r : 0];
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(s[e]) * ar * p.acol[p.per_channel ? col + e : 0];
  store4<OUT>(p.C, 4 * q, v);
}

// ---------------------------------------------------------------------------
// Decode-sized problems (m <= 16): the weights are streamed once, so the
// kernel is bound by HBM, not by the matrix cores.  A workgroup owns NT tiles
// of 16 output channels over all of K; its waves take KC-byte chunks of K in
// turn.  Within a chunk, lane (nl = lane % 16, j = lane / 16) loads the
// 16-byte pieces at k = 64 t + 16 j (t < KC / 64) of weight row nl -- so one
// load instruction reads 64 contiguous bytes of each of 16 rows -- and the
// same pieces of activation row nl (zero for rows >= m), and feeds piece t of
// both to the t-th v_mfma_i32_16x16x64_i8, the weights as the row operand.
// Both operands use the same k bytes per lane, so the k order inside a
// fragment does not matter.  The waves' int32 sums meet in LDS (exact), then
// one pass scales and stores.
// ---------------------------------------------------------------------------
template <int OUT, int NT, int KC, bool STAGED>
__global__ __launch_bounds__(NT == 1 ? 1024 : 512) void k_w8a8_decode(W8A8Problem p) {
  extern __shared__ int red[];   // [waves][NT][256], then (STAGED) [waves][NT][KC / 64][1 KiB]
  constexpr int NP = KC / 64;    // pieces per lane per chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int nl = lane & 15, j = lane >> 4;
  const int K = p.K, nchunks = K / KC;
  const int nt0 = blockIdx.x * NT;
  const bool live = nl < p.M;
  const int8_t *arow = p.A + static_cast<size_t>(live ? nl : 0) * K + 16 * j;
  i32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = i32x4{0, 0, 0, 0};
  // STAGED: the weight chunk goes through this wave's LDS area (NT x 16 rows
  // x KC bytes), loaded as RPI = 1024 / KC rows of KC contiguous bytes per
  // direct-load instruction (lane l: row l / (KC / 16), bytes
  // 16 (l % (KC / 16)), landing in lane order), then read back in the matrix
  // instruction's lane layout; else each load reads 64 bytes of each of 16
  // rows straight into registers.
  constexpr int RPI = 1024 / KC, LPR = KC / 16;
  [[maybe_unused]] char *stage = reinterpret_cast<char *>(red) + nwaves * NT * 256 * 4 + wave * NT * NP * 1024;
  [[maybe_unused]] const auto rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t *>(p.B), 0, static_cast<int>(static_cast<uint32_t>(p.N) * K), 0x00020000);
  [[maybe_unused]] const uint32_t lrow = lane / LPR, lbyte = 16 * (lane % LPR);
  for (int c = wave; c < nchunks; c += nwaves) {
    const int k0 = c * KC;
    i32x4 w[NT][NP];
    if constexpr (STAGED) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of the last chunk are done
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int q = 0; q < NP; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rB, (__attribute__((address_space(3))) void *)(stage + (i * NP + q) * 1024), 16,
              (static_cast<uint32_t>((nt0 + i) * 16 + q * RPI) + lrow) * static_cast<uint32_t>(K) + k0 + lbyte, 0,
              0, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the chunk is in LDS
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int t = 0; t < NP; ++t)
          w[i][t] = *reinterpret_cast<const i32x4 *>(
              stage + (i * NP + nl / RPI) * 1024 + ((nl % RPI) * LPR + 4 * t + j) * 16);
    } else {
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const i32x4 *src = reinterpret_cast<const i32x4 *>(
            p.B + static_cast<size_t>((nt0 + i) * 16 + nl) * K + k0 + 16 * j);
#pragma unroll
        for (int t = 0; t < NP; ++t) w[i][t] = src[4 * t];
      }
    }
    i32x4 a[NP];
#pragma unroll
    for (int t = 0; t < NP; ++t)
      a[t] = live ? *reinterpret_cast<const i32x4 *>(arow + k0 + 64 * t) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < NP; ++t) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[i][t], a[t], acc[i], 0, 0, 0);
  }
  // acc[i][r] of lane l is the sum for activation row l % 16 and channel
  // 16 (nt0 + i) + 4 (l / 16) + r.
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * NT + i) * 256 + r * 64 + lane] = acc[i][r];
  __syncthreads();
  for (int e = threadIdx.x; e < NT * 256; e += blockDim.x) {
    const int i = e >> 8, r = (e >> 6) & 3, l = e & 63;
    const int m = l & 15;
    if (m >= p.M) continue;
    int sum = 0;
    for (int w = 0; w < nwaves; ++w) sum += red[w * NT * 256 + e];
    const int n = (nt0 + i) * 16 + 4 * (l >> 4) + r;
    const float v = static_cast<float>(sum) * p.arow[p.per_token ? m : 0] * p.acol[p.per_channel ? n : 0];
    if constexpr (OUT == QG_FP32) static_cast<float *>(p.C)[static_cast<size_t>(m) * p.N + n] = v;
    else static_cast<uint16_t *>(p.C)[static_cast<size_t>(m) * p.N + n] = f32_to_bits<OUT>(v);
  }
}

namespace {

// Stages (the LDS holds two of the 256 x 256 tile's, three of the 256 x 128
// tile's, four of the smaller ones'), measured at K = 3584 against two:
// 128 x 128 with four, m = 1024, n = 3584: 29.6 -> 22.3 us, m = 512: 24.7 ->
// 16.2 us; 256 x 128 with three, m = 2048, n = 3584: 38.9 -> 34.3 us;
// 64 x 128 with four 5-10 % slower, so it keeps two.
using T256x256 = W8Cfg<256, 256, 2, 4>;      // waves of 128 x 64
using T256x128 = W8Cfg<256, 128, 4, 2, 3>;   // waves of 64 x 64
using T128x128 = W8Cfg<128, 128, 2, 4, 4>;   // waves of 64 x 32
using T64x128 = W8Cfg<64, 128, 2, 4>;        // waves of 32 x 32

struct W8A8Plan {
  int tile;
  int kseg, nsplit;
  size_t bytes;   // int32 partials of a split plan
};

int tiles_of(int M, int N, int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }


// Tile by problem size (below), then K slices when the tiles leave the chip
// mostly idle, each slice at least two steps.  The dispatch override's
// w8a8_split asks for n slices (tests and tuning).
W8A8Plan plan_w8a8(int M, int N, int K) {
  W8A8Plan pl{kT64, 0, 1, 0};
  // Above 64 rows: each of these tiles holds a CU alone, so a launch takes
  // ceil(tiles / CUs) rounds of one tile's time; the tile with the fewest
  // round-weighted tile times wins, ties to the larger tile.  Relative tile
  // times, measured at K = 3584 in one round: 256 x 256 1, 256 x 128 0.63,
  // 128 x 128 0.41.  Against every tile forced, m = 128 .. 4096, n = 3584 and
  // 18944, this picks the fastest (m = 2048, n = 18944: 166.8 us on
  // 256 x 256 where the earlier rule took 128 x 128 at 209.8; m = 256,
  // n = 18944: 33.8 on 256 x 128 against 44.3; m = 512, n = 3584: 20.9 on
  // 128 x 128 against 24.4 on 64 x 128).  Up to 64 rows: 128 x 128 when
  // its tiles fill half the CUs unsplit (four stages beat the smaller
  // tile's two: m = 32, n = 18944, 148 tiles: 18.4 against 26.5 us), else
  // 64 x 128 in K slices (m = 32, n = 3584: 12.3 against 14.9).
  if (M <= 64) {
    if (2 * tiles_of(M, N, 128, 128) >= device_cus()) pl.tile = kT128;
  } else {
    const int cus = device_cus();
    auto cost = [&](int bm, int bn, int w) {
      const long t = tiles_of(M, N, bm, bn);
      return ((t + cus - 1) / cus) * static_cast<long>(w);
    };
    const long c256 = cost(256, 256, 100), c256n = cost(256, 128, 63), c128 = cost(128, 128, 41);
    pl.tile = kT256;
    long best = c256;
    if (c256n < best) { pl.tile = kT256N; best = c256n; }
    if (c128 < best) pl.tile = kT128;
  }
  const int bm = pl.tile == kT64 ? 64 : pl.tile == kT128 ? 128 : 256;
  const int bn = pl.tile == kT256 ? 256 : 128;
  const int tiles = tiles_of(M, N, bm, bn), nsteps = K / 128;
  int want = 1;
  // K slices for launches with few tiles: the 64 x 128 tile (two stages)
  // below 128 tiles, for about 256 workgroups; the larger tiles (three or
  // four stages, faster per step) only below 48 tiles, for about 128 (at
  // m = 512, n = 3584, 112 tiles of 128 x 128: unsplit 20.9 us, three
  // slices 29.6; m = 128, 28 tiles: five slices 15.7, ten 22.6).
  if (pl.tile == kT64) {
    if (tiles < 128 && nsteps >= 4) want = std::min((256 + tiles - 1) / tiles, std::min(nsteps / 2, 16));
  } else if (tiles < 48 && nsteps >= 4) {
    want = std::min((128 + tiles - 1) / tiles, std::min(nsteps / 2, 16));
  }
  if (const int o = dispatch_override().w8a8_split; o > 0) want = std::min(o, nsteps);   // tuning
  {
    if (want >= 2) {
      const int kseg = (nsteps + want - 1) / want;
      pl.kseg = kseg;
      pl.nsplit = (nsteps + kseg - 1) / kseg;
      pl.bytes = static_cast<size_t>(pl.nsplit) * M * N * sizeof(int32_t);
    }
  }
  return pl;
}

template <class Cfg, int OUT>
hipError_t run_w8a8(W8A8Problem p, const W8A8Plan &pl, hipStream_t s) {
  const int tm = (p.M + Cfg::BM - 1) / Cfg::BM, tn = (p.N + Cfg::BN - 1) / Cfg::BN;
  if (p.part) {
    hipLaunchKernelGGL((k_w8a8<Cfg, OUT, true>), dim3(tm * tn * pl.nsplit), dim3(Cfg::NTHR), 0, s, p, tm, tn);
    const long long q = static_cast<long long>(p.M) * p.N / 4;
    hipLaunchKernelGGL(k_w8a8_reduce<OUT>, dim3(static_cast<unsigned>((q + 255) / 256)), dim3(256), 0, s,
                       p, pl.nsplit);
  } else {
    hipLaunchKernelGGL((k_w8a8<Cfg, OUT, false>), dim3(tm * tn), dim3(Cfg::NTHR), 0, s, p, tm, tn);
  }
  return hipGetLastError();
}

template <int OUT>
hipError_t dispatch_w8a8(W8A8Problem p, const W8A8Plan &pl, hipStream_t s) {
  switch (pl.tile) {
    case kT256: return run_w8a8<T256x256, OUT>(p, pl, s);
    case kT256N: return run_w8a8<T256x128, OUT>(p, pl, s);
    case kT128: return run_w8a8<T128x128, OUT>(p, pl, s);
    default: return run_w8a8<T64x128, OUT>(p, pl, s);
  }
}

}  // namespace

// Decode kernel for m <= 16 unless a tile is forced (tests and tuning).
bool w8a8_use_decode(int m) {
  if (dispatch_override().w8a8_tile >= 0) return false;
  return m <= 16;
}

size_t w8a8_workspace_bytes(int m, int n, int k) {
  if (w8a8_use_decode(m)) return 0;
  const W8A8Plan pl = plan_w8a8(m, n, k);
  return pl.nsplit > 1 ? pl.bytes : 0;
}

// Two tiles per workgroup and 256-k chunks once there are many channel tiles
// (more bytes in flight per wave); measured on MI355X at K = 3584: N = 18944,
// m = 1: 23 -> 16 us against one tile and 128-k chunks read as 32 contiguous
// bytes per lane (half-line loads), N = 3584 unchanged within noise.  With
// one tile per workgroup up to 16 waves share K (half the chunks per wave,
// each a memory round trip): N = 3584, m = 1 5.9 -> 4.9 us, m = 16
// 6.3 -> 6.2 us; the two-tile form stays at 8 (16 measured 9-11 % slower).
// From 8 rows (weights under 2 GiB) the weight chunks go through LDS as
// whole 256- or 128-byte row pieces: m = 16, n = 18944 19.9 -> 17.6 us,
// n = 3584 6.2 -> 5.9, bit-equal; at m = 1 no faster (15.9 / 15.8 us at
// n = 18944, 4.9 -> 5.1 at n = 3584), so fewer rows keep the direct loads.
template <int OUT>
hipError_t launch_w8a8_decode(const W8A8Problem &p, hipStream_t s) {
  const int ntiles = p.N >> 4;
  const bool wide = ntiles >= 512 && ntiles % 2 == 0 && p.K % 256 == 0;
  const int nchunks = wide ? p.K >> 8 : p.K >> 7;
  const int maxw = wide ? 8 : 16;
  const int waves = nchunks < maxw ? nchunks : maxw;
  const bool staged = p.M >= 8 && uint64_t(p.N) * p.K < (uint64_t(1) << 31);
  const size_t lds = static_cast<size_t>(waves) * (wide ? 2 : 1) *
                     (256 * sizeof(int) + (staged ? (wide ? 4 : 2) * 1024 : 0));
  if (wide && staged)
    hipLaunchKernelGGL((k_w8a8_decode<OUT, 2, 256, true>), dim3(ntiles / 2), dim3(64 * waves), lds, s, p);
  else if (wide)
    hipLaunchKernelGGL((k_w8a8_decode<OUT, 2, 256, false>), dim3(ntiles / 2), dim3(64 * waves), lds, s, p);
  else if (staged)
    hipLaunchKernelGGL((k_w8a8_decode<OUT, 1, 128, true>), dim3(ntiles), dim3(64 * waves), lds, s, p);
  else
    hipLaunchKernelGGL((k_w8a8_decode<OUT, 1, 128, false>), dim3(ntiles), dim3(64 * waves), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_w8a8(const W8A8Args &a, hipStream_t s) {
  W8A8Plan pl = plan_w8a8(a.M, a.N, a.K);
  W8A8Problem p{a.A, a.B, a.alpha_row, a.alpha_col, a.C, nullptr, a.M, a.N, a.K, a.per_token,
                a.per_channel, 0};
  if (w8a8_use_decode(a.M)) {
    switch (a.out) {
      case QG_FP32: return launch_w8a8_decode<QG_FP32>(p, s);
      case QG_FP16: return launch_w8a8_decode<QG_FP16>(p, s);
      default: return launch_w8a8_decode<QG_BF16>(p, s);
    }
  }
  if (pl.nsplit > 1 && a.ws && a.ws_bytes >= pl.bytes) {
    p.part = static_cast<int32_t *>(a.ws);
    p.kseg = pl.kseg;
  } else {
    pl.nsplit = 1;
  }
  if (const int t = dispatch_override().w8a8_tile; t >= 0) pl.tile = t;   // tests and tuning
  switch (a.out) {
    case QG_FP32: return dispatch_w8a8<QG_FP32>(p, pl, s);
    case QG_FP16: return dispatch_w8a8<QG_FP16>(p, pl, s);
    default: return dispatch_w8a8<QG_BF16>(p, pl, s);
  }
}

}  // namespace qg
