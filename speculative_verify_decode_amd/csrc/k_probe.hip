// A plain streaming read of a device buffer: the practical HBM read ceiling that the step's
// kernels are measured against.  Every 16-byte piece is loaded once with the same
// non-temporal policy the weight and KV streams use; the values are folded into one word
// per thread and stored only if it equals a constant no input makes likely, so the loads
// stay live without adding write traffic worth counting.
#include "sd_common.h"

namespace {

constexpr int kUnroll = 8;  // independent 16-byte loads in flight per thread

// Workgroup w reads the contiguous w-th part of the buffer, 1 KB per wave instruction and
// kUnroll instructions in flight per wave.
__global__ __launch_bounds__(256) void k_read_probe(const u32x4_t* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  size_t i = beg + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * 256 < end; i += kUnroll * 256) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += 256) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(256), 0, st, (const u32x4_t*)src, bytes / 16,
                     sink);
  return hipGetLastError();
}
