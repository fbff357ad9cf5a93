// Streaming-read probe: the rate at which a plain kernel reads device memory on
// this GPU, measured beside the decode kernels as the attainable ceiling next
// to the published HBM peak. Each workgroup reads one contiguous share of the
// buffer with 16-byte loads, PF loads in flight per thread, and folds what it
// read into one word so the loads are not removed.
#include "kvc_device.h"

namespace kvc {
namespace {

constexpr int PROBE_PF = 8;

__global__ __launch_bounds__(WG) void k_read_probe(const u32x4 *buf, int64_t n_vec, int reverse, uint32_t *sink) {
  const int64_t per = (n_vec + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = int64_t(blockIdx.x) * per, b1 = min(n_vec, b0 + per);
  uint32_t x = 0;
  for (int64_t base = b0; base < b1; base += int64_t(WG) * PROBE_PF) {
    u32x4 v[PROBE_PF];
#pragma unroll
    for (int u = 0; u < PROBE_PF; ++u) {
      const int64_t i = base + int64_t(u) * WG + threadIdx.x;
      const bool in = i < b1;
      // reverse: the share [b0, b1) is read from its end; lanes past the share read its first vector
      const int64_t j = !in ? b0 : reverse ? b1 - 1 - (i - b0) : i;
      const u32x4 w = buf[j];
      v[u] = in ? w : u32x4(0u);
    }
#pragma unroll
    for (int u = 0; u < PROBE_PF; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per workgroup: the xor of its threads' words
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= uint32_t(__shfl_xor(int(x), o));
  __shared__ uint32_t wx[WG / 64];
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < WG / 64; ++w) y ^= wx[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace

hipError_t launch_read_probe(const void *buf, size_t bytes, int workgroups, int reverse, uint32_t *sink,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_read_probe, dim3(workgroups), dim3(WG), 0, st, reinterpret_cast<const u32x4 *>(buf),
                     int64_t(bytes / 16), reverse, sink);
  return hipGetLastError();
}

}  // namespace kvc
