// moe.hip -- top-k routed MoE over int4 experts ("acext User Guide (v1.7)",
// 1.2.3 MoE GEMM: fp32 gating logits, expert scales, the routing maps
// expert_for_source_row / expanded_source_row_to_expanded_dest_row, fc1 with a
// gated activation, fc2 into an intermediate buffer, and the weighted
// combine into the final output).
//
// Stages, one launch each:
//   route    one wave per token: top-k of the fp32 logits (ties to the lower
//            expert id) and the softmax over the selected logits;
//   plan     one workgroup: per-expert row counts, offsets, the list of
//            (expert, row range) tiles for the grouped GEMMs, and the
//            permutation token <-> expert-sorted row;
//   fc1      grouped tile GEMM, activation rows gathered through the
//            permutation, gate and up columns in one tile, silu(gate) * up
//            in the epilogue;
//   fc2      grouped tile GEMM over the activation rows;
// The grouped GEMMs use the 256 x 256 direct-load tile (tile_big.hpp) with
// 256-row expert tiles where the shapes allow it, else the 128 x 128 tile
// kernel with 128-row expert tiles.
//   combine  out[t] = sum_j w[t, j] * (y[row(t, j)] + b2[e]), fp32 in rank
//            order.
// Optional parts of runMoe: biased selection logits (route), finished rows
// (route gives them no expert; plan and combine skip their slots), the fc1
// expert biases (fc1 epilogue, before the activation) and the fc2 ones
// (combine), and the normalization mode (route).
#include <mutex>

#include "qg_launch.hpp"
#include "tile_big.hpp"
#include "tile_gemm.hpp"

namespace qg {

// Device scratch of the allocation-free MoE entry point
// (qmoe_grouped_noalloc): the workspace of one call, held by every device the
// library runs on until the process ends.  Host code never passes `scratch`
// itself (on the host that name is a stand-in, not a device address): it
// passes the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kMoeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace {

using CfgMoe = TileCfg<128, 128, 2, 2>;
using CfgMoeDma = DmaCfg<2, 4>;
constexpr int kMoeBM = CfgMoe::BM;   // smallest expert tile (sizes the tile list)

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct MoeLayout {
  size_t ids, wts, row_src, dest, tiles, ntiles, act, y, total;
};

MoeLayout moe_layout(int T, int H, int I, int E, int topk) {
  const size_t R = static_cast<size_t>(T) * topk;
  const size_t max_tiles = (R + kMoeBM - 1) / kMoeBM + E;
  MoeLayout l{};
  size_t o = 0;
  l.ids = o;     o = align_up(o + R * 4);
  l.wts = o;     o = align_up(o + R * 4);
  l.row_src = o; o = align_up(o + R * 4);
  l.dest = o;    o = align_up(o + R * 4);
  l.tiles = o;   o = align_up(o + max_tiles * sizeof(MoeTile));
  l.ntiles = o;  o = align_up(o + 4);
  l.act = o;     o = align_up(o + R * I * 2);
  l.y = o;       o = align_up(o + R * H * 2);
  l.total = o;
  return l;
}

}  // namespace

size_t moe_workspace_bytes(int T, int H, int I, int E, int topk) {
  return moe_layout(T, H, I, E, topk).total;
}

// One wave per token; up to 256 experts (4 logits per lane).  The experts
// are chosen by `sel` (the biased logits when given, else the gating logits)
// and weighted from the gating logits: softmax over the chosen experts
// (renormalize) or over all of them.  A finished row takes no expert.
__global__ __launch_bounds__(256) void k_moe_route(const float *__restrict__ logits,
                                                   const float *__restrict__ sel_logits,
                                                   const uint8_t *__restrict__ finished, int T, int E,
                                                   int topk, int renorm, int32_t *__restrict__ ids,
                                                   float *__restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (finished && finished[t]) {
    if (lane < topk) {
      ids[static_cast<size_t>(t) * topk + lane] = -1;
      wts[static_cast<size_t>(t) * topk + lane] = 0.0f;
    }
    return;
  }
  const float *sl = sel_logits ? sel_logits : logits;
  float v[4], u[4];
  bool cand[4];   // expert lane + 64 i exists and is not chosen yet
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    cand[i] = e < E;
    v[i] = cand[i] ? sl[static_cast<size_t>(t) * E + e] : 0.0f;
    u[i] = cand[i] ? logits[static_cast<size_t>(t) * E + e] : -__builtin_inff();
  }
  float my_l = -__builtin_inff();
  int my_id = 0;
  for (int j = 0; j < topk; ++j) {
    // Lane-local best candidate (strict > keeps the lower expert id on
    // ties), then the wave's best by (value, lower id).  A chosen expert
    // leaves the candidate set, so it cannot win again even when every
    // remaining value is -inf; bi < 0 marks a lane with no candidate.
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (cand[i] && (bi < 0 || v[i] > bv)) { bv = v[i]; bi = lane + 64 * i; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
    }
    // the chosen expert's gating logit, from the lane that holds it
    const int slot = bi >> 6;
    const float mine = slot == 0 ? u[0] : slot == 1 ? u[1] : slot == 2 ? u[2] : u[3];
    const float ul = __shfl(mine, bi & 63);
    if ((bi & 63) == lane) cand[slot] = false;
    if (lane == j) { my_l = ul; my_id = bi; }
  }
  // max and sum over the chosen experts (lanes < topk) or over all experts
  float m = renorm ? my_l : fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float d = 0.0f;
  if (renorm) {
    d = lane < topk ? expf(my_l - m) : 0.0f;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) d += (lane + 64 * i < E) ? expf(u[i] - m) : 0.0f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
  if (lane < topk) {
    ids[static_cast<size_t>(t) * topk + lane] = my_id;
    wts[static_cast<size_t>(t) * topk + lane] = expf(my_l - m) / d;
  }
}

// Single workgroup: counts, offsets, tile list, permutation (the row -> token
// map assembled in LDS and stored in order when it fits).  The exclusive
// scans over experts (rows and tiles) run in one wave, the tile list is
// written by one thread per expert, and rows take their slot within the
// expert through LDS atomics (the order of rows inside an expert does not
// change any output: every row is computed independently).  Each thread
// loads its ids kPlanBatch at a time before using them, so the passes over
// the ids wait for memory once per batch rather than once per row.
constexpr int kPlanBatch = 16;
constexpr int kPlanLdsRows = 16384;   // row -> token map built in LDS up to this many rows
__global__ __launch_bounds__(1024) void k_moe_plan(const int32_t *__restrict__ ids, int R, int E,
                                                   int topk, int bm, MoeTile *__restrict__ tiles,
                                                   int32_t *__restrict__ ntiles,
                                                   int32_t *__restrict__ row_src,
                                                   int32_t *__restrict__ dest) {
  __shared__ int cnt[256], off[256], toff[256], fill[256];
  __shared__ int src_lds[kPlanLdsRows];
  const bool in_lds = R <= kPlanLdsRows;
  const int nthr = blockDim.x;
  for (int e = threadIdx.x; e < 256; e += nthr) { cnt[e] = 0; fill[e] = 0; }
  __syncthreads();
  auto load_batch = [&](int base, int (&e)[kPlanBatch]) {
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) {
      const int r = base + u * nthr + static_cast<int>(threadIdx.x);
      e[u] = r < R ? ids[r] : -1;
    }
  };
  for (int base = 0; base < R; base += kPlanBatch * nthr) {
    int e[kPlanBatch];
    load_batch(base, e);
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u)
      if (e[u] >= 0) atomicAdd(&cnt[e[u]], 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // lane l scans experts 4l .. 4l + 3, then the lanes' totals
    const int lane = threadIdx.x;
    int c[4], t[4], rs = 0, ts = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? cnt[e] : 0;
      t[i] = (c[i] + bm - 1) / bm;
      rs += c[i];
      ts += t[i];
    }
    int ri = rs, ti = ts;   // inclusive scans over lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int ru = __shfl_up(ri, d), tu = __shfl_up(ti, d);
      if (lane >= d) { ri += ru; ti += tu; }
    }
    int ro = ri - rs, to = ti - ts;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) { off[e] = ro; toff[e] = to; }
      ro += c[i];
      to += t[i];
    }
    if (lane == 63) *ntiles = ti;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int r1 = off[e] + cnt[e];
    int k = toff[e];
    for (int r0 = off[e]; r0 < r1; r0 += bm) {
      MoeTile tl;
      tl.expert = e;
      tl.row0 = r0;
      tl.row1 = min(r0 + bm, r1);
      tl.pad = 0;
      tiles[k++] = tl;
    }
  }
  for (int base = 0; base < R; base += kPlanBatch * nthr) {
    int e[kPlanBatch];
    load_batch(base, e);
    // All of the batch's slot claims first (independent LDS atomics, in
    // flight together), then the stores: claiming and storing row by row
    // made each thread wait out one atomic's latency per row (9.8k of the
    // kernel's 18k cycles at 12288 rows).
    int pos[kPlanBatch];
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) pos[u] = e[u] >= 0 ? atomicAdd(&fill[e[u]], 1) : -1;
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) {
      const int r = base + u * nthr + static_cast<int>(threadIdx.x);
      if (r >= R) continue;
      if (e[u] < 0) {   // a finished row's slot: no expert row
        dest[r] = -1;
        continue;
      }
      const int q = off[e[u]] + pos[u];
      if (in_lds) src_lds[q] = r / topk;
      else row_src[q] = r / topk;
      dest[r] = q;
    }
  }
  // Written out in order: scattered 4-byte stores from one workgroup (a
  // cache line per lane) cost more than the LDS round trip.
  if (in_lds) {
    __syncthreads();
    const int rows = off[E - 1] + cnt[E - 1];
    for (int i = threadIdx.x; i < rows; i += nthr) row_src[i] = src_lds[i];
  }
}

// The grid is sized for the most expert tiles routing can produce; the plan
// writes how many there are.  Workgroups past ntiles * tiles_n exit; the
// others (the first ones dispatched, so spread evenly over the XCDs, which
// take workgroup b on XCD b % 8) are renumbered so that each XCD walks a
// contiguous run of (row tile, column tile) pairs: all column tiles of an
// expert row tile then share one XCD's L2 for the tile's activation rows,
// instead of every XCD fetching them (with 8 or 11 column tiles and plain
// order each column tile sat on its own XCD).
__device__ __forceinline__ bool moe_tile_of(const TileProblem &p, int tiles_n, int &tm, int &tn) {
  const int real = *p.ntiles * tiles_n;
  const int b = blockIdx.x;
  if (b >= real) return false;
  const int xcd = b & 7, loc = b >> 3, per = real >> 3, rem = real & 7;
  const int id = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  tm = id / tiles_n;
  tn = id - tm * tiles_n;
  return true;
}

template <int ACT, int MODE>
__global__ __launch_bounds__(CfgMoe::NTHR) void k_moe_gemm(TileProblem p, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int tm, tn;
  if (!moe_tile_of(p, tiles_n, tm, tn)) return;
  tile_gemm<CfgMoe, ACT, 4, MODE>(p, tm, tn, lds);
}

template <int ACT, int MODE>
__global__ __launch_bounds__(CfgMoeDma::NTHR) void k_moe_dma(TileProblem p, int tiles_n) {
  __shared__ __attribute__((aligned(16))) char a0[CfgMoeDma::STAGE_A];
  __shared__ __attribute__((aligned(16))) char a1[CfgMoeDma::STAGE_A];
  __shared__ __attribute__((aligned(16))) char b0[CfgMoeDma::STAGE_B];
  __shared__ __attribute__((aligned(16))) char b1[CfgMoeDma::STAGE_B];
  __shared__ __attribute__((aligned(16))) char sc[2 * CfgMoeDma::SC_WIN];
  int tm, tn;
  if (!moe_tile_of(p, tiles_n, tm, tn)) return;
  const DmaLds L{{a0, a1}, {b0, b1}, sc, nullptr};   // no dense epilogue constants
  tile_gemm_dma<CfgMoeDma, ACT, 4, MODE>(p, tm, tn, L);
}

// out[t, h..h+7] = sum_j w[t, j] * (y[dest[t, j], h..h+7] + b2[e, h..h+7]),
// e = ids[t, j]; slots without an expert row (finished rows) add nothing.
// y is read once and out written once: streaming (nontemporal) accesses
// (measured 2.7 us faster on the 2048-token MoE than plain ones).
template <int ACT>
__global__ __launch_bounds__(256) void k_moe_combine(const uint16_t *__restrict__ y,
                                                     const float *__restrict__ wts,
                                                     const int32_t *__restrict__ dest,
                                                     const int32_t *__restrict__ ids,
                                                     const uint16_t *__restrict__ b2,
                                                     uint16_t *__restrict__ out, int T, int H,
                                                     int topk) {
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per = H >> 3;
  if (idx >= static_cast<long long>(T) * per) return;
  const int t = static_cast<int>(idx / per), h0 = static_cast<int>(idx % per) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const float w = wts[static_cast<size_t>(t) * topk + j];
    const int row = dest[static_cast<size_t>(t) * topk + j];
    if (row < 0) continue;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(y + static_cast<size_t>(row) * H + h0));
    u32x4 b = {0u, 0u, 0u, 0u};
    if (b2) b = *reinterpret_cast<const u32x4 *>(b2 + static_cast<size_t>(ids[static_cast<size_t>(t) * topk + j]) * H + h0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += w * (bits_to_f32<ACT>(static_cast<uint16_t>(v[i] & 0xFFFFu)) +
                         bits_to_f32<ACT>(static_cast<uint16_t>(b[i] & 0xFFFFu)));
      acc[2 * i + 1] += w * (bits_to_f32<ACT>(static_cast<uint16_t>(v[i] >> 16)) +
                             bits_to_f32<ACT>(static_cast<uint16_t>(b[i] >> 16)));
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack2<ACT>(acc[2 * i], acc[2 * i + 1]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + static_cast<size_t>(t) * H + h0));
}

namespace {

template <int ACT>
hipError_t run_moe(const MoeArgs &a, hipStream_t s) {
  const MoeLayout L = moe_layout(a.T, a.H, a.I, a.E, a.topk);
  char *ws = static_cast<char *>(a.ws);
  const int R = a.T * a.topk;
  int32_t *ids = a.ids_out ? a.ids_out : reinterpret_cast<int32_t *>(ws + L.ids);
  float *wts = a.w_out ? a.w_out : reinterpret_cast<float *>(ws + L.wts);
  int32_t *row_src = reinterpret_cast<int32_t *>(ws + L.row_src);
  int32_t *dest = reinterpret_cast<int32_t *>(ws + L.dest);
  MoeTile *tiles = reinterpret_cast<MoeTile *>(ws + L.tiles);
  int32_t *ntiles = reinterpret_cast<int32_t *>(ws + L.ntiles);
  uint16_t *act = reinterpret_cast<uint16_t *>(ws + L.act);
  uint16_t *y = reinterpret_cast<uint16_t *>(ws + L.y);
  // The direct-load tile needs whole 256-column output tiles for fc2, an
  // even number of groups per row (scale/zero pairs), 4-byte aligned scales
  // and zeros, and 32-bit offsets.
  const uintptr_t sz_or = reinterpret_cast<uintptr_t>(a.s1) | reinterpret_cast<uintptr_t>(a.z1) |
                          reinterpret_cast<uintptr_t>(a.s2) | reinterpret_cast<uintptr_t>(a.z2);
  const uint64_t lim = uint64_t(1) << 31;
  const bool dma = a.H % CfgMoeDma::BN == 0 && (a.H / a.group) % 2 == 0 && (a.I / a.group) % 2 == 0 &&
                   (sz_or & 3) == 0 && uint64_t(a.T) * a.H < lim && uint64_t(R) * a.I < lim &&
                   uint64_t(2 * a.I) * a.H / 2 < lim;
  // The dispatch override's moe_tile=S forces the 128 x 128 path (tests and
  // tuning).
  const bool use_dma = dma && !dispatch_override().moe_small_tile;
  const int bm = use_dma ? CfgMoeDma::BM : kMoeBM;
  const int max_tiles = (R + bm - 1) / bm + a.E;

  hipLaunchKernelGGL(k_moe_route, dim3((a.T + 3) / 4), dim3(256), 0, s, a.logits, a.sel_logits,
                     a.finished, a.T, a.E, a.topk, a.renorm, ids, wts);
  hipLaunchKernelGGL(k_moe_plan, dim3(1), dim3(1024), 0, s, ids, R, a.E, a.topk, bm, tiles, ntiles,
                     row_src, dest);

  static std::atomic<uint64_t> attr_fc1{0}, attr_fc2{0};
  if (hipError_t e = set_lds_limit_once(k_moe_gemm<ACT, kMoeFc1>, CfgMoe::LDS, attr_fc1); e != hipSuccess)
    return e;
  if (hipError_t e = set_lds_limit_once(k_moe_gemm<ACT, kMoeFc2>, CfgMoe::LDS, attr_fc2); e != hipSuccess)
    return e;
  TileProblem p1{};
  p1.A = a.x;
  p1.B = a.w1;
  p1.S = a.s1;
  p1.Z = a.z1;
  p1.C = act;
  p1.bias = a.b1;   // [E, 2I] or null, added before the activation
  p1.M = R;
  p1.N = a.I;
  p1.K = a.H;
  p1.group = a.group;
  p1.row_src = row_src;
  p1.tiles = tiles;
  p1.ntiles = ntiles;
  p1.b_expert_stride = static_cast<size_t>(2 * a.I) * (a.H / 2);
  p1.s_expert_stride = static_cast<size_t>(2 * a.I) * (a.H / a.group);
  p1.w_rows = 2 * a.I;
  p1.a_rows = a.T;
  if (use_dma) {
    const int tn1 = a.I / (CfgMoeDma::BN / 2);
    hipLaunchKernelGGL((k_moe_dma<ACT, kMoeFc1>), dim3(max_tiles * tn1), dim3(CfgMoeDma::NTHR), 0, s,
                       p1, tn1);
  } else {
    const int tn1 = a.I / (CfgMoe::BN / 2);
    hipLaunchKernelGGL((k_moe_gemm<ACT, kMoeFc1>), dim3(max_tiles * tn1), dim3(CfgMoe::NTHR),
                       CfgMoe::LDS, s, p1, tn1);
  }

  TileProblem p2{};
  p2.A = act;
  p2.B = a.w2;
  p2.S = a.s2;
  p2.Z = a.z2;
  p2.C = y;
  p2.M = R;
  p2.N = a.H;
  p2.K = a.I;
  p2.group = a.group;
  p2.tiles = tiles;
  p2.ntiles = ntiles;
  p2.b_expert_stride = static_cast<size_t>(a.H) * (a.I / 2);
  p2.s_expert_stride = static_cast<size_t>(a.H) * (a.I / a.group);
  p2.w_rows = a.H;
  p2.a_rows = R;
  if (use_dma) {
    const int tn2 = a.H / CfgMoeDma::BN;
    hipLaunchKernelGGL((k_moe_dma<ACT, kMoeFc2>), dim3(max_tiles * tn2), dim3(CfgMoeDma::NTHR), 0, s,
                       p2, tn2);
  } else {
    const int tn2 = a.H / CfgMoe::BN;
    hipLaunchKernelGGL((k_moe_gemm<ACT, kMoeFc2>), dim3(max_tiles * tn2), dim3(CfgMoe::NTHR),
                       CfgMoe::LDS, s, p2, tn2);
  }

  const long long items = static_cast<long long>(a.T) * (a.H / 8);
  hipLaunchKernelGGL((k_moe_combine<ACT>), dim3(static_cast<unsigned>((items + 255) / 256)),
                     dim3(256), 0, s, y, wts, dest, ids, a.b2, a.out, a.T, a.H, a.topk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe(const MoeArgs &a, hipStream_t s) {
  return a.act == kBF16 ? run_moe<kBF16>(a, s) : run_moe<kFP16>(a, s);
}

// The same launches with the device scratch as the workspace.  Every stage
// writes what a later stage reads (routing maps, tile count and list, fc1
// and fc2 rows) before reading it, so nothing needs clearing between calls.
hipError_t launch_moe_noalloc(MoeArgs a, hipStream_t s) {
  void *ws = nullptr;
  if (hipError_t e = scratch_address(&ws); e != hipSuccess) return e;
  a.ws = ws;
  return launch_moe(a, s);
}

}  // namespace qg
