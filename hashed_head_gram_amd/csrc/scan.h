// Block-wide integer scan shared by the sort, segment and staging kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pg {

// Exclusive scan of one int32 per thread across a block of NT threads
// (integer sums, so any summation order gives the same values): a shuffle
// scan inside each wave, then the wave totals. *total gets the block sum. sh
// holds NT / 64 ints; every thread of the block must call it.
template <int NT>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t x, int32_t* sh,
                                                        int32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int32_t base = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < NT / 64; ++j) {
    const int32_t t = sh[j];
    base += j < w ? t : 0;
    tot += t;
  }
  __syncthreads();   // sh may be reused by the caller after this
  *total = tot;
  return base + v - x;
}

}  // namespace pg
