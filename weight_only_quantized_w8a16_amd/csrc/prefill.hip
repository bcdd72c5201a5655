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
#include <cstdlib>
#include <string>
#include <type_traits>

#include "qg_launch.hpp"
#include "tile_big.hpp"
#include "tile_gemm.hpp"

namespace qg {

// Hardware sends workgroup b to XCD b % 8.  Renumber so each XCD walks a
// contiguous run of tiles in M-major order: neighbours on one XCD share their
// activation rows in that XCD's L2.
__device__ __forceinline__ int xcd_linear_id() {
  const int bid = blockIdx.x, nblk = gridDim.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
}

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

// GS8: int8 codes with one scale per (channel, K-group).
template <class Cfg, int ACT, int WBITS, bool GS8>
__global__ __launch_bounds__(Cfg::NTHR) void k_prefill(TileProblem p, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int id = xcd_linear_id();
  int tm, tn;
  grouped_tile(id, gridDim.x / tiles_n, tiles_n, tm, tn);
  tile_gemm<Cfg, ACT, WBITS, kDense, GS8>(p, tm, tn, lds);
}

template <class Cfg, int ACT, int WBITS, bool GS8>
__global__ __launch_bounds__(Cfg::NTHR) void k_prefill_dma(TileProblem p, int tiles_n) {
  __shared__ __attribute__((aligned(16))) char a0[Cfg::STAGE_A];
  __shared__ __attribute__((aligned(16))) char a1[Cfg::STAGE_A];
  __shared__ __attribute__((aligned(16))) char b0[Cfg::STAGE_B];
  __shared__ __attribute__((aligned(16))) char b1[Cfg::STAGE_B];
  __shared__ __attribute__((aligned(16))) char sc[2 * Cfg::SC_WIN];
  const DmaLds L{{a0, a1}, {b0, b1}, sc};
  const int id = xcd_linear_id();
  int tm, tn;
  grouped_tile(id, gridDim.x / tiles_n, tiles_n, tm, tn);
  tile_gemm_dma<Cfg, ACT, WBITS, kDense, GS8>(p, tm, tn, L);
}

namespace {

using CfgX = TileCfg<256, 256, 2, 4>;   // 8 waves, 128x64 per wave
using CfgD8 = DmaCfg<2, 4>;             // 8 waves, 128x64 per wave, A direct to LDS
using CfgD8N = DmaCfg<4, 2, 128>;       // 256 x 128 tile, 8 waves of 64x64
using CfgD64 = DmaCfg<2, 4, 256, 64>;   // 64 x 256 tile, 8 waves of 32x64
using CfgD128 = DmaCfg<2, 4, 256, 128>; // 128 x 256 tile, 8 waves of 64x64
using CfgL = TileCfg<256, 128, 4, 2>;   // 8 waves, 64x64 per wave
using CfgM = TileCfg<128, 128, 2, 2>;   // 4 waves, 64x64 per wave
using CfgS = TileCfg<64, 64, 2, 2>;     // 4 waves, 32x32 per wave

template <class Cfg, int ACT, int WBITS, bool GS8>
hipError_t run(const GemmArgs &a, hipStream_t s) {
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
  const int tm = (a.M + Cfg::BM - 1) / Cfg::BM, tn = a.N / Cfg::BN;
  auto kern = k_prefill<Cfg, ACT, WBITS, GS8>;
  static bool attr_set = false;   // benign race: idempotent
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(tm * tn), dim3(Cfg::NTHR), Cfg::LDS, s, p, tn);
  return hipGetLastError();
}

template <class Cfg, int ACT, int WBITS, bool GS8>
hipError_t run_dma(const GemmArgs &a, hipStream_t s) {
  // The kernel keeps 32-bit element / byte offsets.
  const uint64_t lim = uint64_t(1) << 31;
  // Otherwise the generic tile kernel of the same width takes the problem.
  using Fallback = std::conditional_t<Cfg::BN == 256, CfgX, CfgL>;
  if (uint64_t(a.M) * a.K >= lim || uint64_t(a.N) * a.K * WBITS / 8 >= lim)
    return run<Fallback, ACT, WBITS, GS8>(a, s);
  // Group scales (and int4 zeros) arrive as 4-byte pairs of groups.
  if ((WBITS == 4 || GS8) &&
      (((a.K / a.group) & 1) != 0 || (reinterpret_cast<uintptr_t>(a.S) & 3) != 0 ||
       (WBITS == 4 && (reinterpret_cast<uintptr_t>(a.Z) & 3) != 0)))
    return run<Fallback, ACT, WBITS, GS8>(a, s);
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
  const int tm = (a.M + Cfg::BM - 1) / Cfg::BM, tn = a.N / Cfg::BN;
  hipLaunchKernelGGL((k_prefill_dma<Cfg, ACT, WBITS, GS8>), dim3(tm * tn), dim3(Cfg::NTHR), 0, s, p, tn);
  return hipGetLastError();
}

// Tile choice, from on-device sweeps at K = 2048 and 3584 (M from 32 to
// 4096): the direct-load tiles once there are enough of them to keep most
// CUs busy, the generic tiles (down to 64 x 64) when the problem would leave
// CUs idle.
// QGEMM_PREFILL_TILE=X|D8|D8N|D64|D128|L|M|S forces one (tests and tuning);
// D8, D8N, D64 and D128 are the 256 x 256, 256 x 128, 64 x 256 and
// 128 x 256 tiles with direct-to-LDS activation loads.
template <int ACT, int WBITS, bool GS8 = false>
hipError_t dispatch(const GemmArgs &a, hipStream_t s) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * (a.N / bn); };
  const bool n256 = a.N % 256 == 0, n128 = a.N % 128 == 0;
  if (const char *o = std::getenv("QGEMM_PREFILL_TILE")) {
    const std::string c(o);
    if (c == "X" && n256) return run<CfgX, ACT, WBITS, GS8>(a, s);
    if (c == "D8" && n256) return run_dma<CfgD8, ACT, WBITS, GS8>(a, s);
    if (c == "D8N" && n128) return run_dma<CfgD8N, ACT, WBITS, GS8>(a, s);
    if (c == "D64" && n256) return run_dma<CfgD64, ACT, WBITS, GS8>(a, s);
    if (c == "D128" && n256) return run_dma<CfgD128, ACT, WBITS, GS8>(a, s);
    if (c == "L" && n128) return run<CfgL, ACT, WBITS, GS8>(a, s);
    if (c == "M" && n128) return run<CfgM, ACT, WBITS, GS8>(a, s);
    if (c == "S") return run<CfgS, ACT, WBITS, GS8>(a, s);
  }
  if (n256 && a.M > 128 && tiles(256, 256) >= 160) return run_dma<CfgD8, ACT, WBITS, GS8>(a, s);
  // Up to 192 rows the 64-row tile wastes fewer rows than a 256-row one.
  if (n256 && a.M > 128 && a.M <= 192 && tiles(64, 256) >= 128) return run_dma<CfgD64, ACT, WBITS, GS8>(a, s);
  if (n128 && a.M > 128 && tiles(256, 128) >= 128) return run_dma<CfgD8N, ACT, WBITS, GS8>(a, s);
  // Fewer rows: shorter direct-load tiles over the full 256-wide weight tile,
  // once there are enough of them.
  if (n256 && a.M <= 64 && tiles(64, 256) >= 256) return run_dma<CfgD64, ACT, WBITS, GS8>(a, s);
  if (n256 && a.M > 64 && a.M <= 128 && tiles(128, 256) >= 256) return run_dma<CfgD128, ACT, WBITS, GS8>(a, s);
  if (n256 && a.M > 128 && tiles(64, 256) >= 128) return run_dma<CfgD64, ACT, WBITS, GS8>(a, s);
  if (n128 && a.M > 128 && tiles(256, 128) >= 200) return run<CfgL, ACT, WBITS, GS8>(a, s);
  if (n128 && a.M > 64 && tiles(128, 128) >= 256) return run<CfgM, ACT, WBITS, GS8>(a, s);
  return run<CfgS, ACT, WBITS, GS8>(a, s);
}

}  // namespace

hipError_t launch_prefill_w4(const GemmArgs &a, hipStream_t s) {
  return a.act == kBF16 ? dispatch<kBF16, 4>(a, s) : dispatch<kFP16, 4>(a, s);
}
hipError_t launch_prefill_w8(const GemmArgs &a, hipStream_t s) {
  if (a.group > 0) return a.act == kBF16 ? dispatch<kBF16, 8, true>(a, s) : dispatch<kFP16, 8, true>(a, s);
  return a.act == kBF16 ? dispatch<kBF16, 8>(a, s) : dispatch<kFP16, 8>(a, s);
}

}  // namespace qg
