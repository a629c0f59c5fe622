// Streaming-read probe (gfx950): the HBM read rate this GPU sustains, the
// measured ceiling the gather and the Engram pass 2 are compared with beside
// the 8 TB/s specification. Every lane reads 16-byte chunks, four in flight,
// over a grid-stride walk; the XOR of what it read goes to one word per block
// so no load can be dropped.
#include "common.h"

namespace pg {

namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(
    const uint4* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i];
    const uint4 b = src[i + stride];
    const uint4 c = src[i + 2 * stride];
    const uint4 d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
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
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pg
