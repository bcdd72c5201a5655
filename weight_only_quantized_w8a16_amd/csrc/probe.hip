// probe.hip -- measurement probes, no part of the method: a plain streaming
// read, the ceiling the HBM-bound kernels are measured against, and an LDS
// read loop, the LDS bandwidth the prefill tiles draw on.  The read probe:  Each thread reads 16-byte pieces with streaming
// (nontemporal) loads; in iteration i workgroup b reads piece
// (i * gridDim + b) * blockDim + thread, so at every moment the grid sweeps one
// contiguous window of the buffer (with the one-pass grid below: two windows,
// the grid's first and second halves of the buffer).  The pieces are XOR-folded and each
// workgroup writes one 32-bit word, so the loads cannot be dropped.
#include "qg_common.hpp"
#include "qg_launch.hpp"

namespace qg {

namespace {
// One pass: enough workgroups that every thread reads exactly kDepth pieces
// (no loop), so the dispatcher keeps replacing finished workgroups with new
// ones and the grid sweeps the buffer front to back.  Measured on MI355X
// (HIP events over back-to-back launches, buffers rotated over 1 GiB) among
// grid-stride, workgroup-chunk and wave-chunk orders with 256 to 1024
// threads, 1 to 8 pieces in flight, 1024 to 8192 or one-pass grids, plain
// and nontemporal loads: 512 threads x 2 pieces, one pass, nontemporal read
// 151 MB in 22.9 us (6.6 TB/s) and 15.4 MB in 4.5 us, the fastest at both
// sizes; grids capped at 4096 workgroups looping over the buffer read 151 MB
// in 24-26 us, and plain loads were 10-20 % slower than nontemporal ones.
constexpr int kProbeThreads = 512;
constexpr unsigned long long kProbeMaxBlocks = 1ull << 22;
constexpr int kDepth = 2;
}  // namespace

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const u32x4 *__restrict__ buf,
                                                              unsigned long long pieces,
                                                              uint32_t *__restrict__ out) {
  __shared__ uint32_t part[kProbeThreads / 64];
  const unsigned long long stride = static_cast<unsigned long long>(gridDim.x) * blockDim.x;
  unsigned long long q = static_cast<unsigned long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // kDepth pieces in flight per thread per iteration.
  for (; q + (kDepth - 1) * stride < pieces; q += kDepth * stride) {
    u32x4 v[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) v[i] = __builtin_nontemporal_load(buf + q + i * stride);
#pragma unroll
    for (int i = 0; i < kDepth; ++i) acc ^= v[i];
  }
  for (; q < pieces; q += stride) acc ^= __builtin_nontemporal_load(buf + q);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

// LDS read probe: each workgroup holds 96 KiB of LDS (one workgroup per CU:
// the CU's 160 KiB hold no second), fills its first 64 KiB, then every
// thread reads 16-byte pieces from it `iters` times -- wave w's read j takes
// the 1 KiB row (7 w + j) % 64, lane l its piece l, so a 16-lane group reads
// 256 consecutive bytes and no two lanes of a group share a bank -- and
// thread 0 writes the shader-clock cycles of the read loop (s_memtime,
// between two barriers).  The pieces are XOR-folded; a fold equal to a fixed
// constant would be written in place of the cycles, so the reads cannot be
// dropped.
template <int NT>
__global__ __launch_bounds__(NT) void k_lds_probe(unsigned long long *__restrict__ cycles, int iters) {
  __shared__ __attribute__((aligned(16))) char lds[96 * 1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4096; i += NT)
    reinterpret_cast<u32x4 *>(lds)[i] = u32x4{uint32_t(i), uint32_t(3 * i), uint32_t(5 * i), uint32_t(7 * i)};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const unsigned long long t0 = __builtin_readcyclecounter();
#pragma unroll 8
  for (int j = 0; j < iters; ++j)
    acc ^= *reinterpret_cast<const u32x4 *>(lds + ((wave * 7 + j) & 63) * 1024 + lane * 16);
  __syncthreads();
  const unsigned long long t1 = __builtin_readcyclecounter();
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) cycles[blockIdx.x] = 0;
  __syncthreads();
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

hipError_t launch_lds_probe(int waves, int iters, int blocks, unsigned long long *cycles, hipStream_t s) {
  switch (waves) {
    case 4: hipLaunchKernelGGL(k_lds_probe<256>, dim3(blocks), dim3(256), 0, s, cycles, iters); break;
    case 8: hipLaunchKernelGGL(k_lds_probe<512>, dim3(blocks), dim3(512), 0, s, cycles, iters); break;
    default: hipLaunchKernelGGL(k_lds_probe<1024>, dim3(blocks), dim3(1024), 0, s, cycles, iters); break;
  }
  return hipGetLastError();
}

size_t read_probe_blocks(size_t bytes) {
  const unsigned long long pieces = bytes / 16;
  const unsigned long long want = (pieces + 1ull * kDepth * kProbeThreads - 1) / (1ull * kDepth * kProbeThreads);
  return want < 1 ? 1 : (want > kProbeMaxBlocks ? kProbeMaxBlocks : static_cast<size_t>(want));
}

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *out, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>(read_probe_blocks(bytes));
  hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4 *>(buf), static_cast<unsigned long long>(bytes / 16), out);
  return hipGetLastError();
}

}  // namespace qg
