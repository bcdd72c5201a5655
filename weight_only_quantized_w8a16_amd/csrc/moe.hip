// moe.hip -- top-k routed MoE over int4 experts ("acext User Guide (v1.7)",
// 1.2.3 MoE GEMM: fp32 gating logits, expert scales, the routing maps
// expert_for_source_row / expanded_source_row_to_expanded_dest_row, fc1 with a
// gated activation, fc2 into an intermediate buffer, and the weighted
// combine into the final output).
//
// Stages, one launch each:
//   route    one wave per token: top-k of the fp32 logits (ties to the lower
//            expert id) and the softmax over the selected logits; per
//            workgroup of 16 tokens also its rows' count per expert and each
//            row's place among them;
//   plan     per-expert row offsets from those counts, the list of (expert,
//            row range) tiles for the grouped GEMMs, and the permutation
//            token <-> expert-sorted row;
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
#include <climits>
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

// Routing: tokens per workgroup (one wave each).
constexpr int kRouteTokens = 16;
// Plan: at most this many workgroups (each reads every routing workgroup's
// counts).
constexpr int kPlanBlocks = 128;

struct MoeLayout {
  size_t ids, wts, row_src, dest, lpos, hist, tiles, ntiles, act, y, total;
};

MoeLayout moe_layout(int T, int H, int I, int E, int topk) {
  const size_t R = static_cast<size_t>(T) * topk;
  const size_t max_tiles = (R + kMoeBM - 1) / kMoeBM + E;
  const size_t nw = (static_cast<size_t>(T) + kRouteTokens - 1) / kRouteTokens;
  MoeLayout l{};
  size_t o = 0;
  l.ids = o;     o = align_up(o + R * 4);
  l.wts = o;     o = align_up(o + R * 4);
  l.row_src = o; o = align_up(o + R * 4);
  l.dest = o;    o = align_up(o + R * 4);
  l.lpos = o;    o = align_up(o + R * 4);
  l.hist = o;    o = align_up(o + nw * E * 4);
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

// Order-preserving integer key of a float: a > b as floats (with -0 == +0)
// exactly when key(a) > key(b) as signed integers; NaNs sort above +inf
// (positive sign) or below -inf (negative), so every value has a place and
// equal keys mean equal values.
__device__ __forceinline__ int order_key(float x) {
  int b = __float_as_int(x);
  if ((b & 0x7FFFFFFF) == 0) b = 0;
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}

// Largest value of x over the wave, by DPP steps inside each 16-lane row
// (quad swaps, then the half-row and row mirrors) and the four row results.
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));   // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));   // row_mirror
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// One wave per token, kRouteTokens tokens per workgroup; up to 256 experts,
// expert lane + 64 i in slot i of a lane.  The experts are chosen by `sel`
// (the biased logits when given, else the gating logits): k times the
// largest remaining value (as an order key: the wave's largest key, then
// the lowest expert id holding it), so ties go to the lower expert id.
// Lane j keeps the j-th choice.  Weights come from the gating logits:
// softmax over the chosen experts (renormalize) or over all of them.  A
// finished row takes no expert.
// For the plan, the workgroup also counts its rows per expert (hist, one
// row of E counts per workgroup) and gives each routed row its place among
// the workgroup's rows of that expert (lpos).  Places are taken with LDS
// atomics, in no fixed order: every expert row is computed on its own, so
// the order of rows within an expert changes no output.
__global__ __launch_bounds__(64 * kRouteTokens) void k_moe_route(
    const float *__restrict__ logits, const float *__restrict__ sel_logits,
    const uint8_t *__restrict__ finished, int T, int E, int topk, int renorm,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ lpos,
    int32_t *__restrict__ hist) {
  __shared__ int h[256];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteTokens + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // This token's logits (loads issued before the counts are cleared).
  const int tc = min(t, T - 1);
  const float *sl = (sel_logits ? sel_logits : logits) + static_cast<size_t>(tc) * E;
  const float *lt = logits + static_cast<size_t>(tc) * E;
  int key[4];
  float u[4];     // gating logits (-inf past E)
  bool cand[4];   // expert exists and is not chosen yet
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    cand[i] = e < E;
    key[i] = order_key(cand[i] ? sl[e] : 0.0f);
    u[i] = cand[i] ? lt[e] : -__builtin_inff();
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  int my_id = -1;   // lanes < topk: the expert of this choice
  if (t < T) {
    if (finished && finished[t]) {
      if (lane < topk) {
        ids[static_cast<size_t>(t) * topk + lane] = -1;
        wts[static_cast<size_t>(t) * topk + lane] = 0.0f;
      }
    } else {
      const int nslot = (E + 63) >> 6;   // slots in use (wave-uniform)
      float my_l = 0.0f, m = -__builtin_inff();
      for (int j = 0; j < topk; ++j) {
        int best = INT_MIN;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (cand[i]) best = max(best, key[i]);
        const int M = wave_max_i32(best);
        // the lowest expert id among the candidates holding key M: slot by
        // slot, the lowest lane (one exists: M is a candidate's key, or every
        // candidate's key is INT_MIN)
        int w = 0;
        float uw = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= nslot) break;
          const unsigned long long hit = __ballot(cand[i] && key[i] == M);
          if (hit) {
            const int src = __builtin_ctzll(hit);
            w = 64 * i + src;
            uw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u[i]), src));
            if (lane == src) cand[i] = false;
            break;
          }
        }
        if (lane == j) { my_id = w; my_l = uw; }
        m = fmaxf(m, uw);
      }
      // Softmax over the chosen experts (max m from the choices, the sum
      // gathered in choice order) or over all of them.
      float d = 0.0f, ex = 0.0f;
      if (renorm) {
        ex = lane < topk ? expf(my_l - m) : 0.0f;
        for (int j = 0; j < topk; ++j)
          d += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
      } else {
        m = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
#pragma unroll
        for (int i = 0; i < 4; ++i) d += (lane + 64 * i < E) ? expf(u[i] - m) : 0.0f;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
        ex = lane < topk ? expf(my_l - m) : 0.0f;
      }
      if (lane < topk) {
        ids[static_cast<size_t>(t) * topk + lane] = my_id;
        wts[static_cast<size_t>(t) * topk + lane] = ex / d;
      }
    }
  }
  if (my_id >= 0) lpos[static_cast<size_t>(t) * topk + lane] = atomicAdd(&h[my_id], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[static_cast<size_t>(blockIdx.x) * E + e] = h[e];
}

// Inclusive prefix sum over the wave's lanes by DPP: sums of four lanes
// inside each 16-lane row (row shifts by 1, 2, 3), of eight and sixteen
// (shifts by 4 and 8 on the upper banks), then the row totals carried into
// the rows above (row broadcasts of lanes 15 and 31).  Lanes shifted in
// from outside a row read 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  int t = x;
  t += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  t += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  t += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xF, 0xF, true);   // row_shr:3
  t += __builtin_amdgcn_update_dpp(0, t, 0x114, 0xF, 0xE, true);   // row_shr:4, lanes 4..15
  t += __builtin_amdgcn_update_dpp(0, t, 0x118, 0xF, 0xC, true);   // row_shr:8, lanes 8..15
  t += __builtin_amdgcn_update_dpp(0, t, 0x142, 0xA, 0xF, true);   // row_bcast:15, rows 1, 3
  t += __builtin_amdgcn_update_dpp(0, t, 0x143, 0xC, 0xF, true);   // row_bcast:31, rows 2, 3
  return t;
}

// Plan: workgroup b handles routing workgroups [b per, (b + 1) per).  Every
// workgroup sums the routing counts per expert over all routing workgroups
// (tot) and over those before its own (pre), scans tot over the experts into
// row and tile offsets, and places its rows: routed row r of expert e goes to
// off[e] + pre[e] + lpos[r].  Workgroup 0 also writes the tile list and its
// length.  The counts (E per routing workgroup) are read once per workgroup.
constexpr int kPlanThreads = 256;
__global__ __launch_bounds__(kPlanThreads) void k_moe_plan(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ lpos,
    const int32_t *__restrict__ hist, int R, int E, int topk, int nw, int per, int bm,
    MoeTile *__restrict__ tiles, int32_t *__restrict__ ntiles, int32_t *__restrict__ row_src,
    int32_t *__restrict__ dest) {
  __shared__ int tot[256], pre[256], off[256], toff[256];
  const int w0 = blockIdx.x * per, w1 = min(nw, w0 + per);
  const int rows_per = kRouteTokens * topk;
  // The first routing workgroup's rows (up to 4 per thread), loaded ahead.
  int e_pre[4], l_pre[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = w0 * rows_per + k * kPlanThreads + static_cast<int>(threadIdx.x);
    const bool ok = k * kPlanThreads + static_cast<int>(threadIdx.x) < rows_per && r < R;
    e_pre[k] = ok ? ids[r] : -2;
    l_pre[k] = ok ? lpos[r] : 0;
  }
  for (int e = threadIdx.x; e < E; e += kPlanThreads) { tot[e] = 0; pre[e] = 0; }
  __syncthreads();
  {
    // Thread (g, e) sums column e over routing workgroups g, g + G, ...
    // (G = 256 / E column groups), 32 loads in flight at a time.
    const int G = kPlanThreads / E;
    const int g = static_cast<int>(threadIdx.x) / E, e = static_cast<int>(threadIdx.x) - g * E;
    if (g < G) {
      constexpr int kBatch = 32;
      int st = 0, sp = 0;
      for (int w = g; w < nw; w += kBatch * G) {
        int v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int wu = w + u * G;
          v[u] = wu < nw ? hist[static_cast<size_t>(wu) * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          st += v[u];
          sp += (w + u * G < w0) ? v[u] : 0;
        }
      }
      atomicAdd(&tot[e], st);
      atomicAdd(&pre[e], sp);
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // lane l scans experts 4l .. 4l + 3, then the lanes' totals
    const int lane = threadIdx.x;
    int c[4], tl[4], rs = 0, ts = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? tot[e] : 0;
      tl[i] = (c[i] + bm - 1) / bm;
      rs += c[i];
      ts += tl[i];
    }
    const int ri = wave_incl_scan(rs), ti = wave_incl_scan(ts);
    int ro = ri - rs, to = ti - ts;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) { off[e] = ro; toff[e] = to; }
      ro += c[i];
      to += tl[i];
    }
    if (lane == 63 && blockIdx.x == 0) *ntiles = ti;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < E; e += kPlanThreads) {
      const int r1 = off[e] + tot[e];
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
  }
  auto place = [&](int r, int e, int lp) {
    if (e < 0) {   // a finished row's slot: no expert row
      dest[r] = -1;
      return;
    }
    const int q = off[e] + pre[e] + lp;
    dest[r] = q;
    row_src[q] = r / topk;
  };
  for (int w = w0; w < w1; ++w) {
    const int r0 = w * rows_per, r1 = min(R, r0 + rows_per);
    if (w == w0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (e_pre[k] != -2) place(w0 * rows_per + k * kPlanThreads + static_cast<int>(threadIdx.x), e_pre[k], l_pre[k]);
    } else {
      for (int r = r0 + static_cast<int>(threadIdx.x); r < r1; r += kPlanThreads) place(r, ids[r], lpos[r]);
    }
    if (w + 1 < w1) {
      __syncthreads();
      for (int e = threadIdx.x; e < E; e += kPlanThreads) pre[e] += hist[static_cast<size_t>(w) * E + e];
      __syncthreads();
    }
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
// One workgroup per token, so the token's weights, rows and experts are
// workgroup-uniform (scalar loads); each thread walks its 8-column pieces of
// the hidden dimension, loading the rows of up to 8 slots together before
// adding them in slot order.  y is read once and out written
// once: streaming (nontemporal) accesses (measured 2.7 us faster on the
// 2048-token MoE than plain ones).
template <int ACT>
__global__ __launch_bounds__(256) void k_moe_combine(const uint16_t *__restrict__ y,
                                                     const float *__restrict__ wts,
                                                     const int32_t *__restrict__ dest,
                                                     const int32_t *__restrict__ ids,
                                                     const uint16_t *__restrict__ b2,
                                                     uint16_t *__restrict__ out, int T, int H,
                                                     int topk) {
  const int t = blockIdx.x;
  constexpr int kBatch = 8;   // slots whose rows are loaded together
  for (int h0 = static_cast<int>(threadIdx.x) * 8; h0 < H; h0 += static_cast<int>(blockDim.x) * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < topk; j0 += kBatch) {
      u32x4 v[kBatch], b[kBatch];
      float w[kBatch];
      int row[kBatch], ex[kBatch];
      bool ok[kBatch];
      // The batch's slot entries first (indexes clamped to the last slot, so
      // the loads are unconditional and go out together), then its rows.
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const size_t q = static_cast<size_t>(t) * topk + min(j0 + u, topk - 1);
        row[u] = dest[q];
        w[u] = wts[q];
        ex[u] = b2 ? ids[q] : 0;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        ok[u] = j0 + u < topk && row[u] >= 0;
        v[u] = b[u] = u32x4{0u, 0u, 0u, 0u};
        if (ok[u]) {
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(y + static_cast<size_t>(row[u]) * H + h0));
          if (b2) b[u] = *reinterpret_cast<const u32x4 *>(b2 + static_cast<size_t>(ex[u]) * H + h0);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (!ok[u]) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += w[u] * (bits_to_f32<ACT>(static_cast<uint16_t>(v[u][i] & 0xFFFFu)) +
                                bits_to_f32<ACT>(static_cast<uint16_t>(b[u][i] & 0xFFFFu)));
          acc[2 * i + 1] += w[u] * (bits_to_f32<ACT>(static_cast<uint16_t>(v[u][i] >> 16)) +
                                    bits_to_f32<ACT>(static_cast<uint16_t>(b[u][i] >> 16)));
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack2<ACT>(acc[2 * i], acc[2 * i + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + static_cast<size_t>(t) * H + h0));
  }
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

  int32_t *lpos = reinterpret_cast<int32_t *>(ws + L.lpos);
  int32_t *hist = reinterpret_cast<int32_t *>(ws + L.hist);
  const int nw = (a.T + kRouteTokens - 1) / kRouteTokens;
  const int nplan = nw < kPlanBlocks ? nw : kPlanBlocks;
  const int per = (nw + nplan - 1) / nplan;
  hipLaunchKernelGGL(k_moe_route, dim3(nw), dim3(64 * kRouteTokens), 0, s, a.logits, a.sel_logits,
                     a.finished, a.T, a.E, a.topk, a.renorm, ids, wts, lpos, hist);
  hipLaunchKernelGGL(k_moe_plan, dim3((nw + per - 1) / per), dim3(kPlanThreads), 0, s, ids, lpos,
                     hist, R, a.E, a.topk, nw, per, bm, tiles, ntiles, row_src, dest);

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

  const int cthreads = a.H / 8 < 256 ? a.H / 8 : 256;
  hipLaunchKernelGGL((k_moe_combine<ACT>), dim3(a.T), dim3(cthreads), 0, s, y, wts, dest, ids, a.b2,
                     a.out, a.T, a.H, a.topk);
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
