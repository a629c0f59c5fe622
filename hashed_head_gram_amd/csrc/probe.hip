// Streaming-read probe (gfx950): the HBM read rate this GPU sustains, the
// measured ceiling the gather and the Engram pass 2 are compared with beside
// the 8 TB/s specification. Each block reads one contiguous chunk of the
// buffer, every lane eight 16-byte loads in flight per round (contiguous
// chunks per block stream from HBM faster than a grid-stride walk, which
// spreads each round over the whole buffer); the XOR of what a block read
// goes to one word per block so no load can be dropped.
#include "common.h"

namespace pg {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(
    const uint4* __restrict__ src, int64_t n16, int64_t chunk, uint32_t* __restrict__ sink) {
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = c0 + chunk < n16 ? c0 + chunk : n16;
  uint32_t acc = 0;
  for (int64_t i = c0 + threadIdx.x; i < c1; i += (int64_t)kProbeThreads * kProbeUnroll) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kProbeThreads;
      v[u] = j < c1 ? src[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) t ^= red[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, int blocks,
                             hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t chunk = (n16 + blocks - 1) / blocks;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(src), n16, chunk, sink);
  return hipGetLastError();
}

}  // namespace pg
