// prefill.hip -- large-M weight-only quantized GEMM (dense tiles) on gfx950.
//
// Above a few rows the weights are reused across many activation rows and
// the matrix cores set the pace, so each workgroup dequantizes its weight
// tile once into LDS and runs bf16/fp16 v_mfma_f32_32x32x16 over it (the
// tile kernel in tile_gemm.hpp).  This is the two-path split the pages
// describe (vllm-omni cpu_int4.py: a dequantize-then-dense-GEMM path for
// multi-row batches; "[Misc][Kernel]: Add GPTQAllSpark Quantization": the
// large-M regime), with the dequantized weight kept on chip instead of
// written back to memory.
#include <type_traits>

#include "qg_launch.hpp"
#include "tile_big.hpp"
#include "tile_dense.hpp"
#include "tile_w8dir.hpp"
#include "tile_gemm.hpp"

namespace qg {

// Hardware sends workgroup b to XCD b % 8.  Renumber so each XCD walks a
// contiguous run of tiles in M-major order: neighbours on one XCD share their
// activation rows in that XCD's L2.
__device__ __forceinline__ int xcd_id(int bid, int nblk) {
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
}
__device__ __forceinline__ int xcd_linear_id() { return xcd_id(blockIdx.x, gridDim.x); }

// Tile of linear position `id` (after the XCD renumbering): groups of up to
// four rows of tiles, walked column by column, so the weight tile of one
// column is used by all row tiles of the group while it is still in L2
// (consecutive positions share an XCD), and the group's activation rows (a
// few MiB) stay resident.
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int &tm, int &tn) {
  constexpr int G = 4;
  const int per_group = G * tiles_n;
  const int first_m = (id / per_group) * G;
  const int gsz = min(G, tiles_m - first_m);
  const int in = id - (id / per_group) * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// A split-K grid is nsplit copies of the tile grid, slice-major: position
// id is tile id % T of K slice id / T (T tiles).
template <bool SPLIT>
__device__ __forceinline__ void split_tile(const TileProblem &p, int tiles_n, int &tm, int &tn,
                                           int &slice) {
  if constexpr (!SPLIT) {
    slice = 0;
    grouped_tile(xcd_linear_id(), gridDim.x / tiles_n, tiles_n, tm, tn);
    return;
  }
  const int nsplit = (p.K / 64 + p.kseg - 1) / p.kseg;
  const int per = gridDim.x / nsplit;
  const int id = xcd_linear_id();
  slice = id / per;
  grouped_tile(id - slice * per, per / tiles_n, tiles_n, tm, tn);
}

// GS8: int8 codes with one scale per (channel, K-group).
template <class Cfg, int ACT, int WBITS, bool GS8>
__global__ __launch_bounds__(Cfg::NTHR) void k_prefill(TileProblem p, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int tm, tn, slice = 0;
  if (p.part) split_tile<true>(p, tiles_n, tm, tn, slice);
  else split_tile<false>(p, tiles_n, tm, tn, slice);
  tile_gemm<Cfg, ACT, WBITS, kDense, GS8>(p, tm, tn, lds, slice);
}

// Split-K reduction: C = RNE(sum of the slices' fp32 partials, in slice
// order (x the channel scale for per-channel int8) + bias), 4 outputs per
// thread.
template <int ACT>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ part, int nsplit,
                                                       int M, int N,
                                                       const uint16_t *__restrict__ colscale,
                                                       const uint16_t *__restrict__ bias,
                                                       int bias_dt, uint16_t *__restrict__ C) {
  const long long q = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= static_cast<long long>(M) * N / 4) return;
  const size_t mn = static_cast<size_t>(M) * N;
  f32x4 acc = *reinterpret_cast<const f32x4 *>(part + 4 * q);
  for (int sl = 1; sl < nsplit; ++sl) acc += *reinterpret_cast<const f32x4 *>(part + sl * mn + 4 * q);
  const int col = static_cast<int>((4 * q) % N);
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float x = acc[2 * h + e];
      if (colscale) x *= bits_to_f32<ACT>(colscale[col + 2 * h + e]);
      if (bias) x += bits_to_f32_dyn(bias[col + 2 * h + e], bias_dt);
      v[e] = x;
    }
    out[h] = pack2<ACT>(v[0], v[1]);
  }
  *reinterpret_cast<uint2 *>(C + 4 * q) = make_uint2(out[0], out[1]);
}

template <class Cfg, int ACT, int WBITS, bool GS8, bool SPLIT, bool PC>
__global__ __launch_bounds__(Cfg::NTHR) void k_prefill_dma(TileProblem p, int tiles_n) {
  __shared__ __attribute__((aligned(16))) char a0[Cfg::STAGE_A];
  __shared__ __attribute__((aligned(16))) char a1[Cfg::STAGE_A];
  __shared__ __attribute__((aligned(16))) char b0[Cfg::STAGE_B];
  __shared__ __attribute__((aligned(16))) char b1[Cfg::STAGE_B];
  __shared__ __attribute__((aligned(16))) char sc[2 * Cfg::SC_WIN];
  __shared__ __attribute__((aligned(16))) char ep[2 * Cfg::BN * 2];
  const DmaLds L{{a0, a1}, {b0, b1}, sc, ep};
  int tm, tn, slice;
  split_tile<SPLIT>(p, tiles_n, tm, tn, slice);
  tile_gemm_dma<Cfg, ACT, WBITS, kDense, GS8, SPLIT, PC>(p, tm, tn, L, slice);
}

// Dequantize-then-dense path, first half: W [N, K] 16-bit row-major into the
// caller's workspace, holding the values the fused tiles put into LDS --
// int4: fma(q, s, z - 8 s) rounded once to the activation type (z = 0
// without zeros; group = K for one scale and zero per channel); int8: the
// codes exactly (the channel scale is applied to the sum), or q * s rounded
// (group scales).
//
// int4: one thread per 8 consecutive k of a row (one tiled 4-byte word), in
// row-major order, so a wave writes one contiguous KiB.  Walking the tiled
// codes in order instead (a wave reading one 1 KiB block of 16 rows and
// writing 16 row pieces, with or without an LDS transpose for the writes)
// measured faster alone (N = 3072, K = 2048: 5.7 against 7.2 us) but slower
// ahead of the dense tile (GEMM + dequant, M = 512: 26.7 against 22.1 us).
template <int ACT>
__global__ __launch_bounds__(256) void k_predequant_w4(const uint8_t *__restrict__ B,
                                                       const uint16_t *__restrict__ S,
                                                       const uint16_t *__restrict__ Z,
                                                       uint16_t *__restrict__ W, int K, int group,
                                                       long long runs) {
  const long long r = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= runs) return;
  const int per_row = K >> 3;
  const int row = static_cast<int>(r / per_row), k0 = static_cast<int>(r % per_row) * 8;
  const uint32_t word = *reinterpret_cast<const uint32_t *>(B + w4_word_offset(row, k0, K));
  const size_t gi = static_cast<size_t>(row) * (K / group) + k0 / group;
  const float sc = bits_to_f32<ACT>(S[gi]);
  const float z8 = (Z ? bits_to_f32<ACT>(Z[gi]) : 0.0f) - 8.0f * sc;
  *reinterpret_cast<u32x4 *>(W + static_cast<size_t>(row) * K + k0) = dequant_word_w4<ACT>(word, sc, z8);
}

// int8: a tiled 1 KiB block holds 16 rows x 64 k; lane l of a block holds
// row l % 16 and the 8-k chunks j and 4 + j (j = l / 16), two 8-byte runs.
// A wave converts one block, read as one contiguous KiB (row-major order,
// one run per thread, measured 17.1 against 9.4 us at N = K = 3584).
template <int ACT, bool GS8>
__device__ __forceinline__ void predequant_w8_piece(u32x4 w, const uint16_t *__restrict__ S, int row,
                                                    int kb0, int K, int group, u32x4 (&out)[2]) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {   // k 32 r + 8 j
    if constexpr (GS8)
      out[r] = dequant_run_w8<ACT>(w[2 * r], w[2 * r + 1],
                                   bits_to_f32<ACT>(S[static_cast<size_t>(row) * (K / group) + (kb0 + 32 * r) / group]));
    else
      out[r] = (ACT == kFP16) ? w8_run_to_f16(w[2 * r], w[2 * r + 1]) : w8_run_to_bf16(w[2 * r], w[2 * r + 1]);
  }
}

// Four consecutive blocks of one 16-row band per workgroup (K a multiple of
// 256): the values are staged in LDS and each row's 256 values leave as
// contiguous 16-byte pieces.
template <int ACT, bool GS8>
__global__ __launch_bounds__(256) void k_predequant_w8(const u32x4 *__restrict__ B,
                                                       const uint16_t *__restrict__ S,
                                                       uint16_t *__restrict__ W, int K, int group) {
  constexpr int KB = 64;
  constexpr int PITCH = 4 * KB * 2 + 16;       // LDS row bytes (padded)
  constexpr int PPR = 4 * KB / 8;              // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) char tile[16 * PITCH];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, nl = l & 15, j = l >> 4;
  const int nkb = K / KB;
  const long long blk0 = static_cast<long long>(blockIdx.x) * 4;   // first block
  const int band = static_cast<int>(blk0 / nkb), kb0 = static_cast<int>(blk0 % nkb) * KB;
  u32x4 out[2];
  predequant_w8_piece<ACT, GS8>(__builtin_nontemporal_load(B + blk0 * 64 + tid), S, band * 16 + nl,
                                kb0 + wave * KB, K, group, out);
#pragma unroll
  for (int e = 0; e < 2; ++e)
    *reinterpret_cast<u32x4 *>(tile + nl * PITCH + (wave * KB + 32 * e + 8 * j) * 2) = out[e];
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 16 * PPR / 256; ++it) {
    const int q = it * 256 + tid, r = q / PPR, c = q % PPR;
    *reinterpret_cast<u32x4 *>(W + static_cast<size_t>(band * 16 + r) * K + kb0 + c * 8) =
        *reinterpret_cast<const u32x4 *>(tile + r * PITCH + c * 16);
  }
}

// int8, any K (a multiple of 64): one block per wave, each lane's values
// written where they belong.
template <int ACT, bool GS8>
__global__ __launch_bounds__(256) void k_predequant_w8_any(const u32x4 *__restrict__ B,
                                                           const uint16_t *__restrict__ S,
                                                           uint16_t *__restrict__ W, int K, int group,
                                                           long long pieces) {
  const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= pieces) return;
  const int nkb = K / 64;
  const long long blk = t >> 6;
  const int l = static_cast<int>(t & 63), nl = l & 15, j = l >> 4;
  const int row = static_cast<int>(blk / nkb) * 16 + nl, kb0 = static_cast<int>(blk % nkb) * 64;
  u32x4 out[2];
  predequant_w8_piece<ACT, GS8>(__builtin_nontemporal_load(B + t), S, row, kb0, K, group, out);
#pragma unroll
  for (int e = 0; e < 2; ++e)
    *reinterpret_cast<u32x4 *>(W + static_cast<size_t>(row) * K + kb0 + 32 * e + 8 * j) = out[e];
}

// Second half: the dense tile over the dequantized weights, tiles in the
// fused tiles' XCD-grouped order.
template <class Cfg, int ACT>
__global__ __launch_bounds__(Cfg::NTHR) void k_dense(DenseProblem p, int tiles_n) {
  constexpr int NA = Cfg::NS > 2 ? Cfg::STAGE_A : 16, NB = Cfg::NS > 2 ? Cfg::STAGE_B : 16;
  constexpr int NA3 = Cfg::NS > 3 ? Cfg::STAGE_A : 16, NB3 = Cfg::NS > 3 ? Cfg::STAGE_B : 16;
  __shared__ __attribute__((aligned(16))) char a0[Cfg::STAGE_A];
  __shared__ __attribute__((aligned(16))) char a1[Cfg::STAGE_A];
  __shared__ __attribute__((aligned(16))) char a2[NA];
  __shared__ __attribute__((aligned(16))) char a3[NA3];
  __shared__ __attribute__((aligned(16))) char b0[Cfg::STAGE_B];
  __shared__ __attribute__((aligned(16))) char b1[Cfg::STAGE_B];
  __shared__ __attribute__((aligned(16))) char b2[NB];
  __shared__ __attribute__((aligned(16))) char b3[NB3];
  const DenseLds L{{a0, a1, a2, a3}, {b0, b1, b2, b3}};
  int tm, tn;
  grouped_tile(xcd_linear_id(), gridDim.x / tiles_n, tiles_n, tm, tn);
  dense_tile_gemm<Cfg, ACT>(p, tm, tn, L);
}

// int8 codes, converted after the LDS read (GS: group scales).
template <class Cfg, int ACT, bool GS, bool SPLIT = false>
__global__ __launch_bounds__(Cfg::NTHR) void k_w8dir(W8DirProblem p, int tiles_n) {
  constexpr int SA = Cfg::STAGE_A, SB = Cfg::STAGE_B;
  __shared__ __attribute__((aligned(16))) char a0[SA];
  __shared__ __attribute__((aligned(16))) char a1[SA];
  __shared__ __attribute__((aligned(16))) char a2[Cfg::NS > 2 ? SA : 16];
  __shared__ __attribute__((aligned(16))) char a3[Cfg::NS > 3 ? SA : 16];
  __shared__ __attribute__((aligned(16))) char b0[SB];
  __shared__ __attribute__((aligned(16))) char b1[SB];
  __shared__ __attribute__((aligned(16))) char b2[Cfg::NS > 2 ? SB : 16];
  __shared__ __attribute__((aligned(16))) char b3[Cfg::NS > 3 ? SB : 16];
  const W8DirLds L{{a0, a1, a2, a3}, {b0, b1, b2, b3}};
  int tm, tn;
  if constexpr (SPLIT) {
    // nsplit copies of the tile grid, slice-major.
    const int nsplit = (p.K / 64 + p.kseg - 1) / p.kseg;
    const int per = gridDim.x / nsplit, id = xcd_linear_id();
    const int slice = id / per;
    grouped_tile(id - slice * per, per / tiles_n, tiles_n, tm, tn);
    w8dir_tile_gemm<Cfg, ACT, GS, true>(p, tm, tn, L, slice);
  } else {
    grouped_tile(xcd_linear_id(), gridDim.x / tiles_n, tiles_n, tm, tn);
    w8dir_tile_gemm<Cfg, ACT, GS>(p, tm, tn, L);
  }
}

// One launch, two fused direct-load tile sizes: the first `big` workgroups
// (whole rounds of the CUs, a multiple of 8) take the first `big` of the
// 256 x 256 tiles, the rest each take a 256 x 128 half of the remaining
// ones, so a last round of large tiles that would leave many CUs idle is cut
// in two.  The halves' stages and scale windows fit in the large tile's LDS
// objects; both sizes give the same bits (same k order and arithmetic).
struct CfgDXBig : DmaCfg<2, 4> {};
struct CfgDXHalf : DmaCfg<4, 2, 128> {};

template <int ACT, int WBITS, bool GS8, bool PC>
__global__ __launch_bounds__(512) void k_prefill_dma_mixed(TileProblem p, int tiles_n, int tiles, int big) {
  using Big = CfgDXBig;
  using Half = CfgDXHalf;
  static_assert(Half::STAGE_A <= Big::STAGE_A && Half::STAGE_B <= Big::STAGE_B && Half::SC_WIN <= Big::SC_WIN &&
                    Half::BN <= Big::BN && Half::NTHR == Big::NTHR && Big::NTHR == 512,
                "half-tile LDS inside the large tile's");
  __shared__ __attribute__((aligned(16))) char a0[Big::STAGE_A];
  __shared__ __attribute__((aligned(16))) char a1[Big::STAGE_A];
  __shared__ __attribute__((aligned(16))) char b0[Big::STAGE_B];
  __shared__ __attribute__((aligned(16))) char b1[Big::STAGE_B];
  __shared__ __attribute__((aligned(16))) char sc[2 * Big::SC_WIN];
  __shared__ __attribute__((aligned(16))) char ep[2 * Big::BN * 2];
  const DmaLds L{{a0, a1}, {b0, b1}, sc, ep};
  const int bid = blockIdx.x;
  int tm, tn;
  if (bid < big) {
    grouped_tile(xcd_id(bid, big), tiles / tiles_n, tiles_n, tm, tn);
    tile_gemm_dma<Big, ACT, WBITS, kDense, GS8, false, PC>(p, tm, tn, L, 0);
    return;
  }
  const int u = xcd_id(bid - big, gridDim.x - big);
  grouped_tile(big + u / 2, tiles / tiles_n, tiles_n, tm, tn);
  tile_gemm_dma<Half, ACT, WBITS, kDense, GS8, false, PC>(p, tm, 2 * tn + (u & 1), L, 0);
}

// One launch, two tile sizes (int8 codes converted after the LDS read): the
// first `big` workgroups (whole rounds of the CUs, a multiple of 8) take the
// first `big` of the 256 x 256 tiles, the rest each take a 128 x 128
// quarter of the remaining ones, so the last, partial round is four times
// as finely cut and ends about when a quarter tile would.  Both sizes share
// the three LDS stages (a quarter tile's stage fits in the front of a large
// one's, each stage still a separate object) and give the fused tiles' bits.
struct CfgWXBig : W8DirCfg<256, 256, 2, 4, 3> {};
struct CfgWXSmall : W8DirCfg<128, 128, 2, 4, 3> {};

template <int ACT, bool GS>
__global__ __launch_bounds__(512) void k_w8dir_mixed(W8DirProblem p, int tiles_n, int tiles, int big) {
  constexpr int SA = CfgWXBig::STAGE_A, SB = CfgWXBig::STAGE_B;
  static_assert(CfgWXSmall::STAGE_A <= SA && CfgWXSmall::STAGE_B <= SB && CfgWXSmall::NS <= CfgWXBig::NS,
                "quarter-tile stages inside the large ones");
  __shared__ __attribute__((aligned(16))) char a0[SA];
  __shared__ __attribute__((aligned(16))) char a1[SA];
  __shared__ __attribute__((aligned(16))) char a2[SA];
  __shared__ __attribute__((aligned(16))) char b0[SB];
  __shared__ __attribute__((aligned(16))) char b1[SB];
  __shared__ __attribute__((aligned(16))) char b2[SB];
  const W8DirLds L{{a0, a1, a2, a2}, {b0, b1, b2, b2}};
  const int bid = blockIdx.x;
  int tm, tn;
  if (bid < big) {
    grouped_tile(xcd_id(bid, big), tiles / tiles_n, tiles_n, tm, tn);
    w8dir_tile_gemm<CfgWXBig, ACT, GS>(p, tm, tn, L);
    return;
  }
  const int u = xcd_id(bid - big, gridDim.x - big);
  grouped_tile(big + u / 4, tiles / tiles_n, tiles_n, tm, tn);
  const int sm = 2 * tm + ((u >> 1) & 1), sn = 2 * tn + (u & 1);
  if (sm * CfgWXSmall::BM >= p.M) return;   // quarter below the last row
  w8dir_tile_gemm<CfgWXSmall, ACT, GS>(p, sm, sn, L);
}

namespace {

using CfgX = TileCfg<256, 256, 2, 4>;   // 8 waves, 128x64 per wave
using CfgD8 = DmaCfg<2, 4>;             // 8 waves, 128x64 per wave, A direct to LDS
using CfgD8N = DmaCfg<4, 2, 128>;       // 256 x 128 tile, 8 waves of 64x64
using CfgD64 = DmaCfg<2, 4, 256, 64>;   // 64 x 256 tile, 8 waves of 32x64
using CfgD128 = DmaCfg<2, 4, 256, 128>; // 128 x 256 tile, 8 waves of 64x64
using CfgL = TileCfg<256, 128, 4, 2>;   // 8 waves, 64x64 per wave
using CfgM = TileCfg<128, 128, 2, 2>;   // 4 waves, 64x64 per wave
// The 64 x 64 tile runs as two K groups of 4 waves (each 32 x 32 per wave,
// half of the K steps, accumulators added through LDS at the end): twice
// the waves for the shapes that leave CUs idle.  Measured against one group:
// M = 512, N = 3072, K = 2048 26.9 -> 25.6 us; M = 128 (two K slices)
// 18.2 -> 15.1 us, M = 64 17.2 -> 14.0 us; W8A16 M = 128, N = 3584 20.4 ->
// 19.4 us; four groups were slower (one workgroup per CU).
using CfgS = TileCfg<64, 64, 2, 2, 2>;
// Dense tiles of the dequantize-then-dense path.
using CfgP256 = DenseCfg<256, 256, 2, 4, 2>;   // 8 waves of 128 x 64, 2 stages
using CfgP128 = DenseCfg<128, 128, 2, 4, 4>;   // 8 waves of 64 x 32, 4 stages
using CfgP64 = DenseCfg<64, 128, 2, 4, 4>;     // 8 waves of 32 x 32, 4 stages
// int8 tiles with the codes converted after the LDS read.
using CfgW256 = W8DirCfg<256, 256, 2, 4, 3>;   // 8 waves of 128 x 64, 3 stages
using CfgW256N = W8DirCfg<256, 128, 4, 2, 3>;  // 8 waves of 64 x 64, 3 stages
using CfgW128 = W8DirCfg<128, 128, 2, 4, 4>;   // 8 waves of 64 x 32, 4 stages
using CfgW64 = W8DirCfg<64, 128, 2, 4, 4>;     // 8 waves of 32 x 32, 4 stages

// K slices of one launch: partials in `part` (nullptr: no split).
struct Split {
  float *part = nullptr;
  int kseg = 0, nsplit = 1;
};

TileProblem dense_problem(const GemmArgs &a, const Split &sp) {
  TileProblem p{};
  p.A = a.A;
  p.B = static_cast<const uint8_t *>(a.B);
  p.S = a.S;
  p.Z = a.Z;
  p.bias = a.bias;
  p.C = a.C;
  p.M = a.M;
  p.N = a.N;
  p.K = a.K;
  p.group = a.group > 0 ? a.group : a.K;
  p.bias_dt = a.bias_dt;
  p.a_rows = a.M;
  p.part = sp.part;
  p.kseg = sp.kseg;
  return p;
}

template <int ACT, int WBITS, bool GS8>
hipError_t reduce_split(const GemmArgs &a, const Split &sp, hipStream_t s) {
  if (!sp.part) return hipGetLastError();
  const long long q = static_cast<long long>(a.M) * a.N / 4;
  hipLaunchKernelGGL(k_splitk_reduce<ACT>, dim3(static_cast<unsigned>((q + 255) / 256)), dim3(256), 0, s,
                     sp.part, sp.nsplit, a.M, a.N, (WBITS == 8 && !GS8) ? a.S : nullptr, a.bias,
                     a.bias_dt, a.C);
  return hipGetLastError();
}

template <class Cfg, int ACT, int WBITS, bool GS8>
hipError_t run(const GemmArgs &a, hipStream_t s, const Split &sp = Split{}) {
  const TileProblem p = dense_problem(a, sp);
  const int tm = (a.M + Cfg::BM - 1) / Cfg::BM, tn = a.N / Cfg::BN;
  auto kern = k_prefill<Cfg, ACT, WBITS, GS8>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = set_lds_limit_once(kern, Cfg::LDS, attr_done); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tm * tn * sp.nsplit), dim3(Cfg::NTHR), Cfg::LDS, s, p, tn);
  return reduce_split<ACT, WBITS, GS8>(a, sp, s);
}

// Whether the direct-load tiles take the problem (else the generic tile of
// the same width does): activation and code bytes below 2 GiB (the buffer
// resources take 31-bit extents and 32-bit offsets), and group scales (int4
// zeros too) in 4-byte pairs of groups.
template <int WBITS, bool GS8, bool PC>
bool dma_ok(const GemmArgs &a) {
  const uint64_t lim = uint64_t(1) << 31;
  if (uint64_t(a.M) * a.K * 2 >= lim || uint64_t(a.N) * a.K * WBITS / 8 >= lim) return false;
  if (((WBITS == 4 && !PC) || GS8) &&
      (((a.K / a.group) & 1) != 0 || (reinterpret_cast<uintptr_t>(a.S) & 3) != 0 ||
       (WBITS == 4 && (reinterpret_cast<uintptr_t>(a.Z) & 3) != 0)))
    return false;
  return true;
}

template <class Cfg, int ACT, int WBITS, bool GS8, bool PC = false>
hipError_t run_dma(const GemmArgs &a, hipStream_t s, const Split &sp = Split{}) {
  using Fallback = std::conditional_t<Cfg::BN == 256, CfgX, CfgL>;
  if (!dma_ok<WBITS, GS8, PC>(a)) return run<Fallback, ACT, WBITS, GS8>(a, s, sp);
  const TileProblem p = dense_problem(a, sp);
  const int tm = (a.M + Cfg::BM - 1) / Cfg::BM, tn = a.N / Cfg::BN;
  if (sp.part)
    hipLaunchKernelGGL((k_prefill_dma<Cfg, ACT, WBITS, GS8, true, PC>), dim3(tm * tn * sp.nsplit),
                       dim3(Cfg::NTHR), 0, s, p, tn);
  else
    hipLaunchKernelGGL((k_prefill_dma<Cfg, ACT, WBITS, GS8, false, PC>), dim3(tm * tn),
                       dim3(Cfg::NTHR), 0, s, p, tn);
  return reduce_split<ACT, WBITS, GS8>(a, sp, s);
}


// Tile shapes.  Choice, from on-device sweeps at K = 2048 and 3584 (M from
// 32 to 4096): the direct-load tiles once there are enough of them to keep
// most CUs busy, the generic tiles (down to 64 x 64) when the problem would
// leave CUs idle.  Every direct-load tile holds a CU alone (its LDS allows no
// second workgroup), so a launch takes ceil(tiles / CUs) rounds of one tile's
// time: above 192 rows, once the 256 x 256 tiles fill half the CUs, the
// choice between them and the 256 x 128 tiles (twice as many, each measured
// at 0.62 of a 256 x 256 tile's time) is the one with fewer round-weighted
// tile times -- e.g. W8A16 M = 512, N = 18944 (148 tiles of 256 x 256: one
// round): 79.6 us against 102.8 on 256 x 128; M = 1024 (296 tiles: two rounds
// against three of 256 x 128): 171.4 against 159.9 us on 256 x 128.  The
// dispatch override's prefill_tile forces one (tests and tuning); D8, D8N,
// D64 and D128 are the 256 x 256, 256 x 128, 64 x 256 and 128 x 256 tiles
// with direct-to-LDS activation loads.

// The fused tiles' choice (the forced fused tile, else by size).
int choose_fused_tile(const GemmArgs &a) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * (a.N / bn); };
  const bool n256 = a.N % 256 == 0, n128 = a.N % 128 == 0;
  switch (dispatch_override().prefill_tile) {
    case kX: if (n256) return kX; break;
    case kD8: if (n256) return kD8; break;
    case kD8N: if (n128) return kD8N; break;
    case kD64: if (n256) return kD64; break;
    case kD128: if (n256) return kD128; break;
    case kL: if (n128) return kL; break;
    case kM: if (n128) return kM; break;
    case kS: return kS;
    default: break;
  }
  if (n256 && a.M > 192) {
    const int cus = device_cus();
    const long t8 = tiles(256, 256);
    if (2 * t8 > cus) {
      const long rounds8 = (t8 + cus - 1) / cus, rounds8n = (2 * t8 + cus - 1) / cus;
      return rounds8n * 62 < rounds8 * 100 ? kD8N : kD8;
    }
  }
  if (n256 && a.M > 128 && tiles(256, 256) >= 160) return kD8;
  // Up to 192 rows the 64-row tile wastes fewer rows than a 256-row one.
  if (n256 && a.M > 128 && a.M <= 192 && tiles(64, 256) >= 128) return kD64;
  if (n128 && a.M > 128 && tiles(256, 128) >= 128) return kD8N;
  // Fewer rows: shorter direct-load tiles over the full 256-wide weight tile,
  // once there are enough of them.
  if (n256 && a.M <= 64 && tiles(64, 256) >= 256) return kD64;
  if (n256 && a.M > 64 && a.M <= 128 && tiles(128, 256) >= 256) return kD128;
  if (n256 && a.M > 128 && tiles(64, 256) >= 128) return kD64;
  if (n128 && a.M > 128 && tiles(256, 128) >= 200) return kL;
  if (n128 && a.M > 64 && tiles(128, 128) >= 256) return kM;
  return kS;
}

// Dequantize-then-dense: the whole weight dequantized once into the
// caller's workspace (N K 16-bit values), then a dense tile; the operands
// must fit its 32-bit buffer offsets.  Taken when forced, and by size where
// the fused tiles would re-dequantize every weight for many row tiles while
// leaving most CUs idle: 512 to 1024 rows, at least 3072 columns (2048
// above 512 rows: M = 1024, N = 2048 28.9 -> 25.0 us; M = 512 equal), fewer
// 256 x 256 tiles than a quarter of the CUs.  Measured on MI355X (dequant + dense
// tile against the fused choice): W4A16 K = 2048, N = 3072: M = 512
// 28.4 -> 21.5 us (64 x 128 tile), M = 1024 31.0 -> 27.1 us (128 x 128);
// W8A16 K = N = 3584, M = 1024: per channel 45.5 -> 43.9 us, group 128
// 56.0 -> 42.6 us.  Slower at M = 256 (20.5 -> 20.7 us), M = 2048
// (36.1 -> 45.4 us) and for N = 13312 or 18944 (M = 512, N = 13312, 104
// tiles: 37.6 -> 65.7 us).
int choose_dense_tile(const GemmArgs &a) {
  const uint64_t lim = uint64_t(1) << 31;
  if (uint64_t(a.M) * a.K * 2 >= lim || uint64_t(a.N) * a.K * 2 >= lim) return -1;
  switch (dispatch_override().prefill_tile) {
    case kP256: return a.N % 256 == 0 ? kP256 : -1;
    case kP128: return a.N % 128 == 0 ? kP128 : -1;
    case kP64: return a.N % 128 == 0 ? kP64 : -1;
    case -1: break;
    default: return -1;   // a fused tile is forced
  }
  const long t8 = static_cast<long>((a.M + 255) / 256) * (a.N / 256);
  if (a.M >= 512 && a.M <= 1024 && (a.N >= 3072 || (a.N >= 2048 && a.M > 512)) && a.N % 128 == 0 &&
      4 * t8 < device_cus())
    return a.M <= 512 ? kP64 : kP128;
  return -1;
}

int choose_tile(const GemmArgs &a) {
  const int d = choose_dense_tile(a);
  return d >= 0 ? d : choose_fused_tile(a);
}

bool is_dense(int tile) { return tile == kP256 || tile == kP128 || tile == kP64; }
size_t dense_bytes(const GemmArgs &a) { return static_cast<size_t>(a.N) * a.K * 2; }

// Split-K plan: K slices written as fp32 partials to the caller's
// workspace, then summed by one reduction launch.  Measured on MI355X, the
// partials' traffic and the extra launch cost about what the shorter K loop
// saves, except on the 64 x 64 tile at up to 128 rows with a long K loop
// (few small tiles, each walking all of K): there two slices gain 15 %
// (M = 128: N = 3072, K = 2048, int4 16.5 -> 13.9 us; N = 3584, K = 3584,
// int8 20.4 -> 17.3 us), while at 256 rows and above, on the larger tiles,
// and once the 64 x 64 tiles alone number 256 or more (M = 128, K = 3584,
// int8, N = 18944: 45 us unsplit, 51 us in two slices; K = 2048, int4,
// N = 13312: 29.5 / 38.8 us, N = 8192: 23.9 / 25.3 us, while N = 4096, 128
// tiles, gains: 23.1 / 18.6 us), splitting was slower.  A slice is a whole number of scale windows
// (8 groups) when the scales come through the direct-load tile's windows,
// a multiple of 8 steps otherwise.  The dispatch override's splitk asks for
// n slices (1: none) on the tile chosen above (tests and tuning).
struct Plan {
  int tile;
  Split split;
  size_t bytes;   // workspace for the partials
};

Plan plan_prefill(const GemmArgs &a, int wbits, bool gs8) {
  Plan pl{choose_tile(a), Split{}, 0};
  if (is_dense(pl.tile)) {
    pl.bytes = dense_bytes(a);
    return pl;
  }
  const int nsteps = a.K / 64;
  const int tiles_s = ((a.M + 63) / 64) * (a.N / 64);
  int want = (pl.tile == kS && a.M <= 128 && nsteps >= 32 && tiles_s < 256) ? 2 : 1;
  if (const int o = dispatch_override().splitk; o > 0) want = o;
  if (want <= 1) return pl;
  const int g = a.group > 0 ? a.group : a.K;
  const bool windows = (wbits == 4 && g != a.K) || gs8;   // scales through LDS windows
  const int unit = windows ? 8 * (g / 64) : 8;
  int kseg = (nsteps + want - 1) / want;
  kseg = (kseg + unit - 1) / unit * unit;
  const int nsplit = (nsteps + kseg - 1) / kseg;
  if (nsplit < 2) return pl;
  pl.split.kseg = kseg;
  pl.split.nsplit = nsplit;
  pl.bytes = static_cast<size_t>(nsplit) * a.M * a.N * sizeof(float);
  return pl;
}

template <int ACT, int WBITS, bool GS8, bool PC>
hipError_t launch_tile(int tile, const GemmArgs &a, hipStream_t s, const Split &sp) {
  switch (tile) {
    case kX: return run<CfgX, ACT, WBITS, GS8>(a, s, sp);
    case kD8: return run_dma<CfgD8, ACT, WBITS, GS8, PC>(a, s, sp);
    case kD8N: return run_dma<CfgD8N, ACT, WBITS, GS8, PC>(a, s, sp);
    case kD64: return run_dma<CfgD64, ACT, WBITS, GS8, PC>(a, s, sp);
    case kD128: return run_dma<CfgD128, ACT, WBITS, GS8, PC>(a, s, sp);
    case kL: return run<CfgL, ACT, WBITS, GS8>(a, s, sp);
    case kM: return run<CfgM, ACT, WBITS, GS8>(a, s, sp);
    default: return run<CfgS, ACT, WBITS, GS8>(a, s, sp);
  }
}

template <class Cfg, int ACT>
hipError_t launch_dense(const DenseProblem &p, hipStream_t s) {
  const int tm = (p.M + Cfg::BM - 1) / Cfg::BM, tn = p.N / Cfg::BN;
  hipLaunchKernelGGL((k_dense<Cfg, ACT>), dim3(tm * tn), dim3(Cfg::NTHR), 0, s, p, tn);
  return hipGetLastError();
}

template <int ACT, int WBITS, bool GS8>
hipError_t run_dense(int tile, const GemmArgs &a, hipStream_t s) {
  uint16_t *W = static_cast<uint16_t *>(a.ws);
  const int grp = a.group > 0 ? a.group : a.K;
  if constexpr (WBITS == 4) {
    const long long runs = static_cast<long long>(a.N) * a.K / 8;
    hipLaunchKernelGGL(k_predequant_w4<ACT>, dim3(static_cast<unsigned>((runs + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint8_t *>(a.B), a.S, a.Z, W, a.K, grp, runs);
  } else {
    const long long pieces = static_cast<long long>(a.N) * a.K / 16;   // 16-byte code pieces
    const unsigned grid = static_cast<unsigned>((pieces + 255) / 256);
    const auto *Bv = static_cast<const u32x4 *>(a.B);
    if (a.K % 256 == 0)
      hipLaunchKernelGGL((k_predequant_w8<ACT, GS8>), dim3(grid), dim3(256), 0, s, Bv, a.S, W, a.K, grp);
    else
      hipLaunchKernelGGL((k_predequant_w8_any<ACT, GS8>), dim3(grid), dim3(256), 0, s, Bv, a.S, W, a.K, grp,
                         pieces);
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const DenseProblem p{a.A, W, (WBITS == 8 && !GS8) ? a.S : nullptr, a.bias, a.bias_dt,
                       a.C, a.M, a.N, a.K};
  switch (tile) {
    case kP256: return launch_dense<CfgP256, ACT>(p, s);
    case kP128: return launch_dense<CfgP128, ACT>(p, s);
    default: return launch_dense<CfgP64, ACT>(p, s);
  }
}

// K slices for the code-converting 64 x 128 tile: 64-k steps per slice, or
// 0 for none.  Forced by the dispatch override's splitk (64 x 128 and
// 128 x 128 tiles); by size for one scale per channel when the 64 x 128
// tiles fill less than half the CUs (up to 128 rows): about one workgroup
// per CU, slices of at least 8 steps, a multiple of 8 (the fused tiles'
// slicing, so that both give the same partials).  Measured on MI355X,
// k = 3584, n = 3584, against the fused 64 x 64 tile in two slices:
// m = 128 18.1 -> 15.8 us (four slices), m = 64 16.5 -> 13.6, m = 32
// 16.2 -> 11.3 (seven); with group scales four slices measured 18.7 against
// 20.7 us at m = 128 but two or seven slower, so those take them only when
// forced.
int w8dir_kseg(const GemmArgs &a, int tile) {
  const int nsteps = a.K / 64;
  int want = 1;
  if (const int o = dispatch_override().splitk; o > 0) {
    want = (tile == kW64 || tile == kW128) ? o : 1;
  } else if (tile == kW64 && a.group <= 0 && a.M <= 128) {
    const int cus = device_cus();
    const long t64 = static_cast<long>((a.M + 63) / 64) * (a.N / 128);
    if (2 * t64 < cus) want = static_cast<int>(std::min<long>(cus / t64, nsteps / 8));
  }
  if (want <= 1) return 0;
  int kseg = (nsteps + want - 1) / want;
  kseg = (kseg + 7) / 8 * 8;
  return (nsteps + kseg - 1) / kseg >= 2 ? kseg : 0;
}
size_t w8dir_bytes(const GemmArgs &a, int kseg) {
  if (kseg <= 0) return 0;
  const int nsplit = (a.K / 64 + kseg - 1) / kseg;
  return static_cast<size_t>(nsplit) * a.M * a.N * sizeof(float);
}

// int8 (channel or group scales), codes converted after the LDS read: the
// tile, or -1 for the other tiles.  The operands must fit 32-bit buffer
// offsets.  By size:
// up to 1024 rows, the 64 x 128 tile when its tiles number between half and
// all of the CUs (one round, most CUs busy), else the 128 x 128 tile on the
// same condition.  Measured on MI355X at K = 3584 (fp16, weights streamed),
// against the other tiles' choice: m = 512, n = 3584 33.5 -> 26.0 us
// (64 x 128); m = 1024, n = 3584 44.4 -> 38.8 us, m = 128, n = 18944
// 52.8 -> 34.4 us (128 x 128); m = 32 / 64, n = 18944 31.1 / 32.9 -> 22.7 /
// 25.5 us (64 x 128).  With fewer tiles up to 128 rows, the 64 x 128 tile
// in K slices (below); unsliced, with fewer tiles (m <= 256, n = 3584,
// 16-21 against 21-30 us) or more than a round of them (m = 256
// and 512, n = 18944; m >= 2048) the other tiles are faster -- except where
// whole rounds of 256 x 256 tiles leave at most a quarter-round of them
// over: then the mixed launch, whose leftover quarters end the last round
// early (m = 1024, k = 3584: n = 18944 180.0 -> 143.9 us, n = 16640
// 177.9 -> 136.7 us against the fused 256 x 256 tile; with more left over,
// m = 1280 or 2048, n = 18944, or n = 22016, and with group scales it
// measured 1-8 % slower than the other tiles' choice).
int choose_w8dir_tile(const GemmArgs &a) {
  const uint64_t lim = uint64_t(1) << 31;
  if (uint64_t(a.M) * a.K * 2 >= lim || uint64_t(a.N) * a.K >= lim) return -1;
  switch (dispatch_override().prefill_tile) {
    case kW256: return a.N % 256 == 0 ? kW256 : -1;
    case kW256N: return a.N % 128 == 0 ? kW256N : -1;
    case kW128: return a.N % 128 == 0 ? kW128 : -1;
    case kW64: return a.N % 128 == 0 ? kW64 : -1;
    case kWX: return a.N % 256 == 0 ? kWX : -1;
    case -1: break;
    default: return -1;   // another tile is forced
  }
  // Group scales (q s rounded per fragment: about 2.5x the conversion work)
  // measured slower than the dequantize-then-dense path at m = 1024,
  // n = 3584, group 128 (44.8 against 41.8 us): forced only.
  if (a.group > 0 || a.N % 128 != 0) return -1;
  const int cus = device_cus();
  if (a.N % 256 == 0) {
    const long t256 = static_cast<long>((a.M + 255) / 256) * (a.N / 256);
    const long full = t256 / cus * cus, rest = t256 - full;
    if (full >= cus && full <= 4L * cus && rest > 0 && 4 * rest <= cus) return kWX;
  }
  if (a.M > 1024) return -1;
  const long t64 = static_cast<long>((a.M + 63) / 64) * (a.N / 128);
  const long t128 = static_cast<long>((a.M + 127) / 128) * (a.N / 128);
  if (2 * t64 >= cus && t64 <= cus) return kW64;
  if (2 * t128 >= cus && t128 <= cus) return kW128;
  if (a.M <= 128 && 2 * t64 < cus && w8dir_kseg(a, kW64) > 0) return kW64;   // in K slices
  return -1;
}

// K slices (kseg > 0, given the workspace): the partials, then the split-K
// reduction (channel scale and bias applied there).
template <class Cfg, int ACT, bool GS>
hipError_t launch_w8dir(const GemmArgs &a, hipStream_t s, int kseg = 0) {
  W8DirProblem p{a.A, static_cast<const uint8_t *>(a.B), a.S, a.bias, a.bias_dt, a.C,
                 a.M, a.N, a.K, GS ? a.group : 0, nullptr, 0};
  const int tm = (a.M + Cfg::BM - 1) / Cfg::BM, tn = a.N / Cfg::BN;
  if (kseg > 0 && a.ws && a.ws_bytes >= w8dir_bytes(a, kseg)) {
    p.part = static_cast<float *>(a.ws);
    p.kseg = kseg;
    const int nsplit = (a.K / 64 + kseg - 1) / kseg;
    hipLaunchKernelGGL((k_w8dir<Cfg, ACT, GS, true>), dim3(tm * tn * nsplit), dim3(Cfg::NTHR), 0, s, p, tn);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    return reduce_split<ACT, 8, GS>(a, Split{p.part, kseg, nsplit}, s);
  }
  hipLaunchKernelGGL((k_w8dir<Cfg, ACT, GS>), dim3(tm * tn), dim3(Cfg::NTHR), 0, s, p, tn);
  return hipGetLastError();
}

// The mixed launch: whole rounds of 256 x 256 tiles when chosen by size,
// half the large tiles (rounded down to a multiple of 8) when forced.
template <int ACT, bool GS>
hipError_t launch_w8dir_mixed(const GemmArgs &a, hipStream_t s) {
  const W8DirProblem p{a.A, static_cast<const uint8_t *>(a.B), a.S, a.bias, a.bias_dt, a.C,
                       a.M, a.N, a.K, GS ? a.group : 0, nullptr, 0};
  const int tiles_n = a.N / 256, tiles = ((a.M + 255) / 256) * tiles_n;
  const int cus = device_cus();
  const int big = dispatch_override().prefill_tile == kWX ? tiles / 2 / 8 * 8 : tiles / cus * cus;
  hipLaunchKernelGGL((k_w8dir_mixed<ACT, GS>), dim3(big + 4 * (tiles - big)), dim3(512), 0, s, p, tiles_n,
                     tiles, big);
  return hipGetLastError();
}

template <int ACT, bool GS>
hipError_t run_w8dir(int tile, const GemmArgs &a, hipStream_t s) {
  switch (tile) {
    case kWX: return launch_w8dir_mixed<ACT, GS>(a, s);
    case kW256: return launch_w8dir<CfgW256, ACT, GS>(a, s);
    case kW256N: return launch_w8dir<CfgW256N, ACT, GS>(a, s);
    case kW128: return launch_w8dir<CfgW128, ACT, GS>(a, s, w8dir_kseg(a, kW128));
    default: return launch_w8dir<CfgW64, ACT, GS>(a, s, w8dir_kseg(a, kW64));
  }
}

// The mixed fused launch (256 x 256 tiles for whole rounds, 256 x 128
// halves for the rest): the number of large-tile workgroups, or -1 when not
// taken.  By size, where its cost in the tile-choice model (a round of large
// tiles 100, of halves 62) undercuts either tile alone: m = 1024, n = 18944,
// one round of each against three of halves.  Measured on MI355X against
// the 256 x 128 tile: int8 group 128, k = 3584: n = 18944 189.7 -> 176.0 us,
// n = 16640 181.6 -> 173.5; int4 g64, k = 2048: n = 18944 111.5 -> 99.9,
// n = 16640 105.6 -> 97.3; int4 per channel n = 18944 105.9 -> 97.5; where
// the model says no (m = 2048, n = 13312) it measured 8 % slower.  Forced:
// half the large tiles.  Never with forced K slices.
int dma_mixed_big(const GemmArgs &a) {
  const auto &o = dispatch_override();
  const bool forced = o.prefill_tile == kDX;
  if ((!forced && o.prefill_tile != -1) || o.splitk > 1 || a.N % 256 != 0) return -1;
  const long t8 = static_cast<long>((a.M + 255) / 256) * (a.N / 256);
  if (forced) return static_cast<int>(t8 / 2 / 8 * 8);
  const int cus = device_cus();
  const long full = t8 / cus * cus, rest = t8 - full;
  if (full < cus || rest == 0) return -1;
  const long rounds8 = (t8 + cus - 1) / cus, rounds8n = (2 * t8 + cus - 1) / cus;
  const long mixed = full / cus * 100 + (2 * rest + cus - 1) / cus * 62;
  return mixed < std::min(rounds8 * 100, rounds8n * 62) ? static_cast<int>(full) : -1;
}

template <int ACT, int WBITS, bool GS8, bool PC>
hipError_t run_dma_mixed(const GemmArgs &a, int big, hipStream_t s) {
  const TileProblem p = dense_problem(a, Split{});
  const int tiles_n = a.N / 256, tiles = ((a.M + 255) / 256) * tiles_n;
  hipLaunchKernelGGL((k_prefill_dma_mixed<ACT, WBITS, GS8, PC>), dim3(big + 2 * (tiles - big)), dim3(512), 0, s,
                     p, tiles_n, tiles, big);
  return hipGetLastError();
}

template <int ACT, int WBITS, bool GS8 = false, bool PC = false>
hipError_t dispatch(const GemmArgs &a, hipStream_t s) {
  if constexpr (WBITS == 8) {
    if (const int w = choose_w8dir_tile(a); w >= 0) return run_w8dir<ACT, GS8>(w, a, s);
  }
  if (const int big = dma_mixed_big(a); big >= 0 && dma_ok<WBITS, GS8, PC>(a))
    return run_dma_mixed<ACT, WBITS, GS8, PC>(a, big, s);
  Plan pl = plan_prefill(a, WBITS, GS8);
  if (is_dense(pl.tile)) {
    if (a.ws && a.ws_bytes >= pl.bytes) return run_dense<ACT, WBITS, GS8>(pl.tile, a, s);
    // Too little workspace: the fused tiles, as if no dense tile were chosen.
    GemmArgs b = a;
    b.ws = nullptr;
    b.ws_bytes = 0;
    return launch_tile<ACT, WBITS, GS8, PC>(choose_fused_tile(a), b, s, Split{});
  }
  if (pl.split.nsplit > 1 && a.ws && a.ws_bytes >= pl.bytes)
    pl.split.part = static_cast<float *>(a.ws);
  else
    pl.split = Split{};
  return launch_tile<ACT, WBITS, GS8, PC>(pl.tile, a, s, pl.split);
}

}  // namespace

size_t prefill_workspace_bytes(const GemmArgs &a, int wbits) {
  if (wbits == 8)
    if (const int w = choose_w8dir_tile(a); w >= 0) return w8dir_bytes(a, w8dir_kseg(a, w));
  const Plan pl = plan_prefill(a, wbits, wbits == 8 && a.group > 0);
  return (pl.split.nsplit > 1 || is_dense(pl.tile)) ? pl.bytes : 0;
}

hipError_t launch_prefill_w4(const GemmArgs &a, hipStream_t s) {
  if (a.group == a.K)   // one scale and zero per channel
    return a.act == kBF16 ? dispatch<kBF16, 4, false, true>(a, s) : dispatch<kFP16, 4, false, true>(a, s);
  return a.act == kBF16 ? dispatch<kBF16, 4>(a, s) : dispatch<kFP16, 4>(a, s);
}
hipError_t launch_prefill_w8(const GemmArgs &a, hipStream_t s) {
  if (a.group > 0) return a.act == kBF16 ? dispatch<kBF16, 8, true>(a, s) : dispatch<kFP16, 8, true>(a, s);
  return a.act == kBF16 ? dispatch<kBF16, 8>(a, s) : dispatch<kFP16, 8>(a, s);
}

}  // namespace qg
