// Device fill of large synthetic inputs with the counter-based generator of
// the synth module: element i of a stream is built from
//     word = mix64(base + (i + 1) * 0x9E3779B97F4A7C15)
// (output i of a splitmix64 generator started at `base`; base is computed
// by the host from the seed and stream id). Normal-like values: sum of the
// word's four 16-bit fields minus 131070, times an fp32 scale (one rounding),
// optionally rounded to bf16 (nearest even). NF4 codes are the words' bytes;
// NF4 scales are fp16(fp32(q16 + 49152) * fp32(0.05/65536)).
// Input generation only: none of the n-gram memory's arithmetic is here.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

// Every product is rounded to fp32 on its own before any conversion: no
// contraction into fused multiply-add or mixed-precision multiply-convert
// instructions, which would round once and change rounding ties.
#pragma clang fp contract(off)

namespace {

__device__ __forceinline__ uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t gen_word(uint64_t base, uint64_t i) {
  return sm_mix(base + (i + 1) * 0x9E3779B97F4A7C15ull);
}

__device__ __forceinline__ float gen_normal(uint64_t w, float scale) {
  const int32_t s = (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) +
                    (int32_t)((w >> 32) & 0xFFFF) + (int32_t)(w >> 48) - 131070;
  return __fmul_rn((float)s, scale);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_normal_kernel(void* dst, int64_t n, uint64_t base, float scale,
                                   int32_t bf16, int64_t offset) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = gen_normal(gen_word(base, (uint64_t)(offset + i)), scale);
    if (bf16)
      static_cast<uint16_t*>(dst)[i] = to_bf16(v);
    else
      static_cast<float*>(dst)[i] = v;
  }
}

__global__ void fill_words_kernel(uint64_t* dst, int64_t n_words, uint64_t base) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride)
    dst[i] = gen_word(base, (uint64_t)i);
}

__global__ void fill_nf4_scales_kernel(__half* dst, int64_t n, uint64_t base) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const float c = 0.05f / 65536.0f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t q = (uint32_t)(gen_word(base, (uint64_t)i) & 0xFFFF);
    float prod = __fmul_rn((float)q + 49152.0f, c);
    // Keep the fp32 product: without this the backend folds the multiply and
    // the fp16 conversion into one mixed-precision op that rounds only once.
    asm volatile("" : "+v"(prod));
    dst[i] = __float2half_rn(prod);
  }
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int synth_fill_normal(void* dst, int64_t n,
                                                             uint64_t base, float scale,
                                                             int32_t bf16, int64_t offset,
                                                             hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(n)), dim3(256), 0, s, dst, n, base,
                     scale, bf16, offset);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

__attribute__((visibility("default"))) int synth_fill_words(void* dst, int64_t n_words,
                                                            uint64_t base, hipStream_t s) {
  if (n_words <= 0) return 0;
  hipLaunchKernelGGL(fill_words_kernel, dim3(grid_for(n_words)), dim3(256), 0, s,
                     static_cast<uint64_t*>(dst), n_words, base);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

__attribute__((visibility("default"))) int synth_fill_nf4_scales(void* dst, int64_t n,
                                                                 uint64_t base,
                                                                 hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_nf4_scales_kernel, dim3(grid_for(n)), dim3(256), 0, s,
                     static_cast<__half*>(dst), n, base);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
