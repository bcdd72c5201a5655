// qg_launch.hpp -- host-side launchers implemented in the .hip translation
// units and called by the C ABI layer (api.cpp) after validation.  Every
// launcher assumes its arguments were validated and returns the HIP status
// of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace qg {

// Raises a kernel's dynamic-LDS limit to `bytes` once per device (the
// attribute belongs to the current device's copy of the kernel): `done`
// holds one bit per device id, set after a successful call.  Concurrent
// first calls may both set it, which is harmless.
template <class Kern>
hipError_t set_lds_limit_once(Kern kern, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Compute units of the current device (cached per device; 256 if unknown).
inline int device_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

// Dispatch override (qg_set_override): forced choices, or the automatic
// ones (kPathAuto, -1, 0, false).  A forced tile or path that does not fit a
// problem is ignored for that problem.
enum { kPathAuto = 0, kPathDecode = 1, kPathPrefill = 2 };
// Prefill tiles (prefill.hip), in the order qg_set_override names them.
// kP256 .. kP64: the dense tiles of the dequantize-then-dense path.
// kW256 .. kW64: the int8 per-channel tiles that convert codes after the LDS read;
// kWX: 256 x 256 ones for whole rounds of the CUs, 128 x 128 quarters for the rest;
// kDX: fused 256 x 256 tiles for whole rounds, 256 x 128 halves for the rest.
enum PrefillTile { kX, kD8, kD8N, kD64, kD128, kL, kM, kS, kP256, kP128, kP64, kW256, kW256N, kW128, kW64, kWX, kDX };
// W8A8 tiles (w8a8.hip), in the order qg_set_override names them.
enum W8A8Tile { kT256, kT256N, kT128, kT64 };
struct Override {
  int path = kPathAuto;
  int prefill_tile = -1;       // PrefillTile, or -1
  int splitk = 0;              // prefill K slices (1: none), or 0
  bool moe_small_tile = false; // MoE grouped GEMMs on the 128 x 128 tile
  int w8a8_tile = -1;          // W8A8Tile, or -1
  int w8a8_split = 0;          // W8A8 K slices, or 0
};
Override dispatch_override();

hipError_t launch_repack_w4(const uint8_t *src, uint8_t *dst, int n, int k, hipStream_t s);
hipError_t launch_unrepack_w4(const uint8_t *src, uint8_t *dst, int n, int k, hipStream_t s);
hipError_t launch_repack_w8(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s);
hipError_t launch_unrepack_w8(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s);
hipError_t launch_repack_w8_kn(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s);
hipError_t launch_unrepack_w8_kn(const int8_t *src, int8_t *dst, int n, int k, hipStream_t s);

hipError_t launch_quantize_w4(const void *W, uint8_t *packed, void *scale, void *zero, int n,
                              int k, int group, int w_dt, int sz_dt, hipStream_t s);

hipError_t launch_dequant_w4(const uint8_t *B, const uint16_t *S, const uint16_t *Z, void *W,
                             int n, int k, int group, int act, int out, hipStream_t s);
hipError_t launch_dequant_w8(const int8_t *B, const uint16_t *S, void *W, int n, int k, int group,
                             int act, int out, hipStream_t s);

// Dense GEMM problem as the kernels see it.
struct GemmArgs {
  const uint16_t *A;      // [M, K]
  const void *B;          // tiled codes
  const uint16_t *S;      // scales
  const uint16_t *Z;      // zeros (w4) or null
  const uint16_t *bias;   // [N] or null
  uint16_t *C;            // [M, N]
  int M, N, K, group;     // group: 64/128 (w4; w8 with group scales), 0 = per channel (w8)
  int act, bias_dt;
  void *ws = nullptr;     // caller's workspace (split-K partials), may be null
  size_t ws_bytes = 0;
};

// Decode path: M <= 16, weights streamed once.
hipError_t launch_decode_w4(const GemmArgs &a, hipStream_t s);
hipError_t launch_decode_w8(const GemmArgs &a, hipStream_t s);
// Prefill path: any M, matrix-core tiles with weights dequantized into LDS.
hipError_t launch_prefill_w4(const GemmArgs &a, hipStream_t s);
// Workspace bytes the prefill path would use for split-K on this problem (0:
// none); with less workspace it runs unsplit.
size_t prefill_workspace_bytes(const GemmArgs &a, int wbits);
hipError_t launch_prefill_w8(const GemmArgs &a, hipStream_t s);

// MoE pipeline.
struct MoeArgs {
  const uint16_t *x;
  const float *logits;
  const uint8_t *w1;
  const uint16_t *s1, *z1;
  const uint8_t *w2;
  const uint16_t *s2, *z2;
  uint16_t *out;
  int T, H, I, E, topk, group, act;
  int32_t *ids_out;
  float *w_out;
  void *ws;
  // optional parts of runMoe (null / 1 for the plain call)
  const float *sel_logits = nullptr;    // [T, E] biased logits that choose the experts
  const uint8_t *finished = nullptr;    // [T], nonzero: no expert, zero output
  const uint16_t *b1 = nullptr;         // [E, 2I] fc1 biases
  const uint16_t *b2 = nullptr;         // [E, H] fc2 biases
  int renorm = 1;                       // 1: renormalize over the chosen experts
};
size_t moe_workspace_bytes(int T, int H, int I, int E, int topk);
hipError_t launch_moe(const MoeArgs &a, hipStream_t s);
// Allocation-free MoE: the workspace is the library's device scratch of
// kMoeScratchBytes (moe.hip); callers check the problem fits first.
constexpr size_t kMoeScratchBytes = size_t(64) << 20;
hipError_t launch_moe_noalloc(MoeArgs a, hipStream_t s);

}  // namespace qg

namespace qg {

// W8A8 (int8 activations x int8 weights, fp32 row/column scales).
struct W8A8Args {
  const int8_t *A;          // [M, K]
  const int8_t *B;          // [N, K]
  const float *alpha_row;   // [M] if per_token else [1]
  const float *alpha_col;   // [N] if per_channel else [1]
  void *C;                  // [M, N] in `out`
  int M, N, K;
  int per_token, per_channel;
  int out;                  // QG_BF16, QG_FP16 or QG_FP32
  void *ws;                 // split-K partials, may be null
  size_t ws_bytes;
};
// Workspace bytes the W8A8 kernels would use (split-K), 0 if none; with
// less they run unsplit.
size_t w8a8_workspace_bytes(int m, int n, int k);
hipError_t launch_w8a8(const W8A8Args &a, hipStream_t s);

}  // namespace qg

namespace qg {

// Quantized embedding lookup.
struct EmbedArgs {
  const int32_t *ids;       // [tokens]
  int tokens;
  const void *B;            // table codes, tiled or portable
  int tiled;                // 1: the GEMM's tiled layout; 0: portable
  int bits;                 // 4 or 8
  const uint16_t *S, *Z;    // scales, zeros (int4, may be null)
  void *out;                // [tokens, hidden] in out_dt
  int vocab, hidden;
  int group;                // int4: 64, 128 or hidden; int8: 0 (per row), 64 or 128
  int act, out_dt;
};
hipError_t launch_embed(const EmbedArgs &a, hipStream_t s);

}  // namespace qg

namespace qg {

// Streaming-read probe (measurement).
size_t read_probe_blocks(size_t bytes);
hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *out, hipStream_t s);
hipError_t launch_lds_probe(int waves, int iters, int blocks, unsigned long long *cycles, hipStream_t s);

}  // namespace qg
