// Backward pass of the scalar-gated path and the sparse row-wise table update
// (gfx950). PageGram tech report §3.3 (row-wise RMS optimiser with replayed
// decay), §9.1 (beta2 = 0.95) and §9.4 check 4 (sparse gradient == dense).
//
//   de = g dy W                 (projection GEMM, fp32 out)
//   dW = g dy^T e               (split-K GEMM over tokens, fp32 partials,
//                                reduced in split order)
//   table gradient: lookups (t, n, k) sorted by row with a stable LSD radix
//   sort (4-bit digits), then a 16-lane group per distinct row sums
//   s_{t,n,k} (.) de[t][(n,k) slice] over its lookups in sorted order, which
//   is lookup order (stable sort); rows with more than 16 lookups (hot
//   n-grams: a few hundred lookups under Zipf text) go to a whole block each,
//   summed per lane group and then across groups in a fixed order --
//   deterministic either way, no atomics on values.
//   step: 16 lanes per distinct row apply the replayed decay of the steps
//   the row missed and the RMS step of this one.
#include "common.h"
#include "scan.h"

namespace pg {
namespace {

constexpr int kThreads = 256;
constexpr int kRadixBits = 4;
constexpr int kDigits = 1 << kRadixBits;
constexpr int kItems = 8;                          // items per thread
constexpr int kTile = kThreads * kItems;           // items per block


// ---------------------------------------------------------------------------
// Transpose (bf16): out[c][r] = in[r][c] for r < rows, 0 for rows <= r < rows_pad.

__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(
    const uint16_t* __restrict__ in, int64_t rows, int64_t cols, int64_t ld_in,
    uint16_t* __restrict__ out, int64_t rows_pad, int64_t ld_out) {
  __shared__ uint16_t t[64][66];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int rr = ty + 4 * q;
    const int64_t r = r0 + rr, c = c0 + tx;
    t[rr][tx] = (r < rows && c < cols) ? in[r * ld_in + c] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int cc = ty + 4 * q;
    const int64_t c = c0 + cc, r = r0 + tx;
    if (c < cols && r < rows_pad) out[c * ld_out + r] = t[tx][cc];
  }
}

// The same with 16-byte accesses: a 64 x 64 tile read as rows of eight
// 16-byte chunks, written as columns of eight. cols, ld_in, rows_pad and
// ld_out multiples of 8 and both pointers 16-byte aligned (checked by the
// launcher).
__global__ __launch_bounds__(kThreads) void transpose_bf16_v8_kernel(
    const uint16_t* __restrict__ in, int64_t rows, int64_t cols, int64_t ld_in,
    uint16_t* __restrict__ out, int64_t rows_pad, int64_t ld_out) {
  __shared__ __attribute__((aligned(16))) uint16_t t[64][72];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = threadIdx.x + q * kThreads;
    const int rr = idx >> 3, cc = (idx & 7) * 8;
    const int64_t r = r0 + rr, c = c0 + cc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows && c < cols) v = *reinterpret_cast<const uint4*>(in + r * ld_in + c);
    *reinterpret_cast<uint4*>(&t[rr][cc]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = threadIdx.x + q * kThreads;
    const int cc = idx >> 3, rr = (idx & 7) * 8;
    const int64_t c = c0 + cc, r = r0 + rr;
    if (c < cols && r < rows_pad) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)t[rr + 2 * j][cc] | ((uint32_t)t[rr + 2 * j + 1][cc] << 16);
      *reinterpret_cast<uint4*>(out + c * ld_out + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// out[i] = sum_{s < splits} part[s * n + i], summed in s order.
__global__ __launch_bounds__(kThreads) void reduce_splits_kernel(
    const float* __restrict__ part, int splits, int64_t n, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) acc += part[(int64_t)s * n + i];
    out[i] = acc;
  }
}

// ---------------------------------------------------------------------------
// Stable LSD radix sort of (uint32 key, int32 value) pairs, 4-bit digits.
// Block b owns items [b * kTile, (b+1) * kTile); thread t of it owns the
// kItems consecutive items starting at b * kTile + t * kItems.

// keys[i] (row as uint32) and vals[i] = i for the lookups; clears the
// long-segment counter used by the segment reduction.
__global__ __launch_bounds__(kThreads) void sort_init_kernel(
    const int64_t* __restrict__ rows, int64_t n, uint32_t* __restrict__ keys,
    int32_t* __restrict__ vals, int32_t* __restrict__ n_long) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_long = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    keys[i] = (uint32_t)rows[i];
    vals[i] = (int32_t)i;
  }
}

// counts[d * nblk + b] = number of block b's keys with digit d.
__global__ __launch_bounds__(kThreads) void radix_hist_kernel(
    const uint32_t* __restrict__ keys, int64_t n, int shift, int32_t* __restrict__ counts) {
  __shared__ int32_t c[kDigits];
  if (threadIdx.x < kDigits) c[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int64_t i = base + q;
    if (i < n) atomicAdd(&c[(keys[i] >> shift) & (kDigits - 1)], 1);
  }
  __syncthreads();
  if (threadIdx.x < kDigits) counts[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = c[threadIdx.x];
}

// In-place exclusive scan of m int32 values by one block; total -> *total.
__global__ __launch_bounds__(kThreads) void scan_small_kernel(int32_t* __restrict__ a, int64_t m,
                                                             int32_t* __restrict__ total) {
  __shared__ int32_t sh[kThreads / 64];
  const int64_t per = (m + kThreads - 1) / kThreads;
  const int64_t lo = threadIdx.x * per, hi = lo + per < m ? lo + per : m;
  int32_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += a[i];
  int32_t tot;
  int32_t run = block_exclusive_scan<kThreads>(s, sh, &tot);
  if (total && threadIdx.x == 0) *total = tot;
  for (int64_t i = lo; i < hi; ++i) {
    const int32_t v = a[i];
    a[i] = run;
    run += v;
  }
}

// Stable scatter of one digit pass; offs = scanned counts (digit-major).
__global__ __launch_bounds__(kThreads) void radix_scatter_kernel(
    const uint32_t* __restrict__ kin, const int32_t* __restrict__ vin, int64_t n, int shift,
    const int32_t* __restrict__ offs, uint32_t* __restrict__ kout, int32_t* __restrict__ vout) {
  __shared__ int32_t F[kDigits * kThreads];       // [digit][thread] counts, then prefixes
  __shared__ int32_t sh[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)t * kItems;
  uint32_t k[kItems];
  int32_t v[kItems];
  int dg[kItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int64_t i = base + q;
    const bool live = i < n;
    k[q] = live ? kin[i] : 0u;
    v[q] = live ? vin[i] : 0;
    dg[q] = live ? (int)((k[q] >> shift) & (kDigits - 1)) : -1;
  }
#pragma unroll
  for (int d = 0; d < kDigits; ++d) {
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < kItems; ++q) cnt += dg[q] == d;
    F[d * kThreads + t] = cnt;
  }
  __syncthreads();
  // exclusive scan of F (digit-major, kDigits * kThreads entries): thread j
  // owns kDigits consecutive entries, all of digit j * kDigits / kThreads
  int32_t loc[kDigits];
  int32_t run = 0;
#pragma unroll
  for (int q = 0; q < kDigits; ++q) {
    loc[q] = run;
    run += F[t * kDigits + q];
  }
  int32_t tot;
  const int32_t before = block_exclusive_scan<kThreads>(run, sh, &tot);
#pragma unroll
  for (int q = 0; q < kDigits; ++q) F[t * kDigits + q] = loc[q] + before;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    if (dg[q] < 0) continue;
    const int d = dg[q];
    int rank = 0;
#pragma unroll
    for (int p = 0; p < q; ++p) rank += dg[p] == d;
    const int64_t pos = (int64_t)offs[(int64_t)d * gridDim.x + blockIdx.x] +
                        (F[d * kThreads + t] - F[d * kThreads]) + rank;
    kout[pos] = k[q];
    vout[pos] = v[q];
  }
}

// ---------------------------------------------------------------------------
// Segments of equal keys in the sorted array.

// flags[i] = 1 where a new key starts; per-block sums -> bsum[b].
__global__ __launch_bounds__(kThreads) void seg_flags_kernel(
    const uint32_t* __restrict__ keys, int64_t n, int32_t* __restrict__ flags,
    int32_t* __restrict__ bsum) {
  __shared__ int32_t s[kThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
  int32_t c = 0;
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int64_t i = base + q;
    if (i < n) {
      const int32_t f = (i == 0 || keys[i] != keys[i - 1]) ? 1 : 0;
      flags[i] = f;
      c += f;
    }
  }
  int32_t tot;
  block_exclusive_scan<kThreads>(c, s, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

// Segment id of every head; seg_start[id] = its position; the last block
// also writes the sentinel seg_start[n_unique] = n and *n_unique.
__global__ __launch_bounds__(kThreads) void seg_starts_kernel(
    const int32_t* __restrict__ flags, int64_t n, const int32_t* __restrict__ boff,
    const int32_t* __restrict__ total, int32_t* __restrict__ seg_start,
    int64_t* __restrict__ n_unique) {
  __shared__ int32_t s[kThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
  int32_t c = 0;
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int64_t i = base + q;
    if (i < n) c += flags[i];
  }
  int32_t tot;
  int32_t id = boff[blockIdx.x] + block_exclusive_scan<kThreads>(c, s, &tot);
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int64_t i = base + q;
    if (i < n && flags[i]) seg_start[id++] = (int32_t)i;
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    seg_start[*total] = (int32_t)n;
    *n_unique = *total;
  }
}

// Per-row gradient sums. A row's lookups are contiguous in the sorted
// order; ugrad[s][0..r) = sum over them, in that order, of sign (.) de slice.
// Lanes of a 16-lane group cover V-element chunks of the row (V = 4 when
// r % 4 == 0, else 1): chunk c0 + lane, c0 + 16 + lane, ...
constexpr int kRowLanes = 16;
constexpr int kGroups = kThreads / kRowLanes;      // lane groups per block
constexpr int kShortMax = 16;                      // longest segment of one group

template <int V>
__device__ __forceinline__ void load_chunk(const float* __restrict__ p, float (&x)[V]) {
  if constexpr (V == 4) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
  } else {
    x[0] = *p;
  }
}

template <int V>
__device__ __forceinline__ void store_chunk(float* __restrict__ p, const float (&x)[V]) {
  if constexpr (V == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  } else {
    *p = x[0];
  }
}

// acc += sign (.) x, where bits holds the V sign bits of the chunk (bit set:
// negate); the chunk never crosses a 64-bit sign word since V divides 64.
template <int V>
__device__ __forceinline__ void add_signed(float (&acc)[V], const float (&x)[V], uint32_t bits) {
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] += ((bits >> v) & 1u) ? -x[v] : x[v];
}

// One group per segment of at most kShortMax lookups: each lane fetches one
// lookup index, the group broadcasts them and keeps four row loads in
// flight. Longer segments are appended to long_list (after the counter at
// long_list[0]) for seg_reduce_long_kernel.
template <int V>
__global__ __launch_bounds__(kThreads) void seg_reduce_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ vals,
    const int32_t* __restrict__ seg_start, const int64_t* __restrict__ n_unique, int OK, int r,
    int W, int use_signs, const float* __restrict__ de, const uint64_t* __restrict__ signs,
    int64_t* __restrict__ urows, float* __restrict__ ugrad, int32_t* __restrict__ long_list) {
  const int64_t sidx = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kRowLanes;
  const int ln = threadIdx.x % kRowLanes;
  const int gbase = (int)(threadIdx.x % 64) - ln;   // first lane of the group in its wave
  if (sidx >= *n_unique) return;                    // the whole group leaves together
  const int32_t i0 = seg_start[sidx], i1 = seg_start[sidx + 1];
  const int len = i1 - i0;
  if (ln == 0) urows[sidx] = (int64_t)keys[i0];
  if (len > kShortMax) {
    if (ln == 0) long_list[1 + atomicAdd(long_list, 1)] = (int32_t)sidx;
    return;
  }
  const int64_t E = (int64_t)OK * r;
  const uint32_t q = ln < len ? (uint32_t)vals[i0 + ln] : 0u;
  const uint32_t tok = q / (uint32_t)OK;
  const int64_t base = (int64_t)tok * E + (int64_t)(q - tok * (uint32_t)OK) * r;
  const int nc = r / V;
  for (int c0 = 0; c0 < nc; c0 += kRowLanes) {     // trip count uniform in the group
    const int c = c0 + ln;
    const bool act = c < nc;
    const int j = act ? c * V : 0;
    float acc[V] = {};
    for (int k = 0; k < len; k += 4) {             // len uniform in the group
      float x[4][V];
      uint32_t sb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t b = __shfl(base, gbase + ((k + u) & 15), 64);
        const uint32_t qq = __shfl(q, gbase + ((k + u) & 15), 64);
        sb[u] = 0u;
#pragma unroll
        for (int v = 0; v < V; ++v) x[u][v] = 0.f;
        if (act && k + u < len) {
          load_chunk<V>(de + b + j, x[u]);
          if (use_signs)
            sb[u] = (uint32_t)(signs[(int64_t)qq * W + (j >> 6)] >> (j & 63)) & ((1u << V) - 1u);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (k + u < len) add_signed<V>(acc, x[u], sb[u]);
    }
    if (act) store_chunk<V>(ugrad + sidx * r + j, acc);
  }
}

// One block per long segment (list from seg_reduce_kernel; entries in any
// order, each summed by one block in a fixed order): the block stages up to
// 256 lookups at a time in LDS, group g sums lookups g, g + 16, ... of the
// segment in order, then group 0 adds the 16 group sums in group order.
template <int V>
__global__ __launch_bounds__(kThreads) void seg_reduce_long_kernel(
    const int32_t* __restrict__ vals, const int32_t* __restrict__ seg_start,
    const int32_t* __restrict__ long_list, int OK, int r, int W, int use_signs,
    const float* __restrict__ de, const uint64_t* __restrict__ signs,
    float* __restrict__ ugrad) {
  __shared__ int64_t sbase[kThreads];
  __shared__ uint32_t sq[kThreads];
  __shared__ float red[kGroups][kRowLanes][V];
  const int grp = threadIdx.x / kRowLanes, ln = threadIdx.x % kRowLanes;
  const int n_long = long_list[0];
  const int64_t E = (int64_t)OK * r;
  const int nc = r / V;
  for (int li = blockIdx.x; li < n_long; li += gridDim.x) {     // uniform in the block
    const int64_t sidx = long_list[1 + li];
    const int32_t i0 = seg_start[sidx], i1 = seg_start[sidx + 1];
    for (int c0 = 0; c0 < nc; c0 += kRowLanes) {
      const int c = c0 + ln;
      const bool act = c < nc;
      const int j = act ? c * V : 0;
      float acc[V] = {};
      for (int32_t b0 = i0; b0 < i1; b0 += kThreads) {
        __syncthreads();                            // previous batch fully read
        const int32_t i = b0 + (int32_t)threadIdx.x;
        if (i < i1) {
          const uint32_t q = (uint32_t)vals[i];
          const uint32_t tok = q / (uint32_t)OK;
          sbase[threadIdx.x] = (int64_t)tok * E + (int64_t)(q - tok * (uint32_t)OK) * r;
          sq[threadIdx.x] = q;
        }
        __syncthreads();
        const int cnt = i1 - b0 < kThreads ? i1 - b0 : kThreads;
        for (int k = grp; k < cnt; k += 4 * kGroups) {
          float x[4][V];
          uint32_t sb[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int e = k + u * kGroups;
            sb[u] = 0u;
#pragma unroll
            for (int v = 0; v < V; ++v) x[u][v] = 0.f;
            if (act && e < cnt) {
              load_chunk<V>(de + sbase[e] + j, x[u]);
              if (use_signs)
                sb[u] = (uint32_t)(signs[(int64_t)sq[e] * W + (j >> 6)] >> (j & 63)) &
                        ((1u << V) - 1u);
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (k + u * kGroups < cnt) add_signed<V>(acc, x[u], sb[u]);
        }
      }
#pragma unroll
      for (int v = 0; v < V; ++v) red[grp][ln][v] = acc[v];
      __syncthreads();
      if (grp == 0 && act) {
        float sum[V] = {};
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int v = 0; v < V; ++v) sum[v] += red[g][ln][v];
        store_chunk<V>(ugrad + sidx * r + j, sum);
      }
      __syncthreads();                              // red reused by the next chunk
    }
  }
}

// ---------------------------------------------------------------------------
// Row-wise RMS step and flush.

// sum over the 16 lanes of a row group (fixed xor tree: deterministic)
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int sh = kRowLanes / 2; sh >= 1; sh >>= 1) x += __shfl_xor(x, sh, 64);
  return x;
}

__global__ __launch_bounds__(kThreads) void rms_step_kernel(
    const int64_t* __restrict__ urows, const float* __restrict__ ugrad,
    const int64_t* __restrict__ n_unique, int r, float* __restrict__ table,
    float* __restrict__ vhat, int64_t* __restrict__ last, int64_t step, float lr, float beta2,
    float wd, float eps) {
  const int64_t sidx = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kRowLanes;
  const int ln = threadIdx.x % kRowLanes;
  // every lane of a 16-lane group takes part in the group sum: a group past
  // n_unique computes on row 0 of its own (unwritten) slot range and stores
  // nothing
  const bool live = sidx < *n_unique;
  const int64_t row = live ? urows[sidx] : 0;
  const float* g = ugrad + (live ? sidx : 0) * r;
  float ss = 0.f;
  for (int j = ln; j < r; j += kRowLanes) ss += live ? g[j] * g[j] : 0.f;
  const float m = group_sum(ss) / (float)r;
  if (!live) return;
  int64_t k = step - last[row];
  if (k < 1) k = 1;
  const float v = powf(beta2, (float)k) * vhat[row] + (1.0f - beta2) * m;
  const float decay = powf(1.0f - lr * wd, (float)k);
  const float inv = lr / (sqrtf(v) + eps);
  float* th = table + row * r;
  for (int j = ln; j < r; j += kRowLanes) th[j] = th[j] * decay - inv * g[j];
  if (ln == 0) {
    vhat[row] = v;
    last[row] = step;
  }
}

__global__ __launch_bounds__(kThreads) void rms_flush_kernel(
    int64_t R, int r, float* __restrict__ table, float* __restrict__ vhat,
    int64_t* __restrict__ last, int64_t step, float lr, float beta2, float wd) {
  for (int64_t row = (int64_t)blockIdx.x * kThreads + threadIdx.x; row < R;
       row += (int64_t)gridDim.x * kThreads) {
    const int64_t k = step - last[row];
    if (k <= 0) continue;
    const float decay = powf(1.0f - lr * wd, (float)k);
    float* th = table + row * r;
    for (int j = 0; j < r; ++j) th[j] *= decay;
    vhat[row] *= powf(beta2, (float)k);
    last[row] = step;
  }
}

__global__ void set_i64_kernel(int64_t* p, int64_t v) { *p = v; }

int64_t al(int64_t x) { return (x + 255) / 256 * 256; }

// out[c][r] = in[r][c] (zeros for rows <= r < rows_pad), 16-byte accesses
// where the shapes and pointers allow.
void transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld_in,
                    uint16_t* out, int64_t rows_pad, int64_t ld_out, hipStream_t s) {
  const dim3 grid((unsigned)((rows_pad + 63) / 64), (unsigned)((cols + 63) / 64));
  const bool v8 = cols % 8 == 0 && ld_in % 8 == 0 && rows_pad % 8 == 0 && ld_out % 8 == 0 &&
                  ((uintptr_t)in & 15) == 0 && ((uintptr_t)out & 15) == 0;
  if (v8)
    hipLaunchKernelGGL(transpose_bf16_v8_kernel, grid, dim3(kThreads), 0, s, in, rows, cols,
                       ld_in, out, rows_pad, ld_out);
  else
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(kThreads), 0, s, in, rows, cols, ld_in,
                       out, rows_pad, ld_out);
}

unsigned grid_for(int64_t n, int64_t per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > 1048576) b = 1048576;
  return (unsigned)b;
}

}  // namespace

// Geometry of the backward workspace.
BackwardPlan backward_plan(int64_t N, int64_t d, int64_t E, int64_t L) {
  BackwardPlan p{};
  const int64_t tiles = ((d + 255) / 256) * ((E + 255) / 256);
  const int64_t kblk = (N + 63) / 64;              // 64-token K stages
  int64_t splits = (256 + tiles - 1) / tiles;
  if (splits > kblk) splits = kblk;
  if (splits < 1) splits = 1;
  const int64_t per = (kblk + splits - 1) / splits;
  p.splits = (int)((kblk + per - 1) / per);
  p.kc = (int)(per * 64);
  p.kpad = (int64_t)p.splits * p.kc;
  p.nblk = (L + kTile - 1) / kTile;
  int64_t off = 0;
  p.off_dyT = off; off += al(d * p.kpad * 2);
  p.off_eT = off;  off += al(E * p.kpad * 2);
  p.off_WT = off;  off += al(E * d * 2);
  p.off_part = off; off += al((int64_t)p.splits * d * E * 4);
  p.off_k0 = off; off += al(L * 4);
  p.off_k1 = off; off += al(L * 4);
  p.off_v0 = off; off += al(L * 4);
  p.off_v1 = off; off += al(L * 4);
  p.off_counts = off; off += al((kDigits * p.nblk + 16) * 4);
  p.off_flags = off; off += al(L * 4);
  p.off_seg = off; off += al((L + 1) * 4);
  p.off_long = off; off += al((L / (kShortMax + 1) + 2) * 4);
  p.bytes = off;
  return p;
}

hipError_t launch_backward_scalar(const DevLayout& Ly, const BackwardPlan& p, float g,
                                  const int64_t* rows, const uint64_t* signs, const void* e,
                                  const void* dy, const void* W, int64_t N, int64_t d,
                                  float* dW, float* de, int64_t* urows, float* ugrad,
                                  int64_t* n_unique, void* workspace, hipStream_t s) {
  const int OK = Ly.O * Ly.K;
  const int r = Ly.r;
  const int64_t E = (int64_t)OK * r;
  const int64_t L = N * OK;
  auto* ws = static_cast<uint8_t*>(workspace);
  auto* dyT = reinterpret_cast<uint16_t*>(ws + p.off_dyT);
  auto* eT = reinterpret_cast<uint16_t*>(ws + p.off_eT);
  auto* WT = reinterpret_cast<uint16_t*>(ws + p.off_WT);
  auto* part = reinterpret_cast<float*>(ws + p.off_part);
  auto* k0 = reinterpret_cast<uint32_t*>(ws + p.off_k0);
  auto* k1 = reinterpret_cast<uint32_t*>(ws + p.off_k1);
  auto* v0 = reinterpret_cast<int32_t*>(ws + p.off_v0);
  auto* v1 = reinterpret_cast<int32_t*>(ws + p.off_v1);
  auto* counts = reinterpret_cast<int32_t*>(ws + p.off_counts);
  auto* total = counts + kDigits * p.nblk;
  auto* flags = reinterpret_cast<int32_t*>(ws + p.off_flags);
  auto* seg = reinterpret_cast<int32_t*>(ws + p.off_seg);
  auto* long_list = reinterpret_cast<int32_t*>(ws + p.off_long);
  const auto* dyb = static_cast<const uint16_t*>(dy);
  const auto* eb = static_cast<const uint16_t*>(e);
  const auto* Wb = static_cast<const uint16_t*>(W);

  // de = g dy W: A = dy [N][d], B = W^T [E][d]
  transpose_bf16(Wb, d, E, E, WT, d, d, s);
  hipError_t err = launch_gemm_f32(dy, (int)d, WT, (int)d, N, (int)E, (int)d, 1, g, de, E, s);
  if (err != hipSuccess) return err;
  // dW = g dy^T e: A = dy^T [d][kpad], B = e^T [E][kpad], split K
  transpose_bf16(dyb, N, d, d, dyT, p.kpad, p.kpad, s);
  transpose_bf16(eb, N, E, E, eT, p.kpad, p.kpad, s);
  err = launch_gemm_f32(dyT, (int)p.kpad, eT, (int)p.kpad, d, (int)E, p.kc, p.splits, g, part, E, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3(grid_for(d * E, kThreads)), dim3(kThreads), 0, s,
                     part, p.splits, d * E, dW);

  // sort the lookups by row (stable), digits of the row index up to R
  hipLaunchKernelGGL(sort_init_kernel, dim3(grid_for(L, kThreads)), dim3(kThreads), 0, s, rows,
                     L, k0, v0, long_list);
  int bits = 1;
  while (bits < 32 && ((uint64_t)1 << bits) < (uint64_t)Ly.n_rows) ++bits;
  uint32_t* ka = k0;
  uint32_t* kb = k1;
  int32_t* va = v0;
  int32_t* vb = v1;
  for (int shift = 0; shift < bits; shift += kRadixBits) {
    hipLaunchKernelGGL(radix_hist_kernel, dim3((unsigned)p.nblk), dim3(kThreads), 0, s, ka, L,
                       shift, counts);
    hipLaunchKernelGGL(scan_small_kernel, dim3(1), dim3(kThreads), 0, s, counts,
                       (int64_t)kDigits * p.nblk, total);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3((unsigned)p.nblk), dim3(kThreads), 0, s, ka, va,
                       L, shift, counts, kb, vb);
    uint32_t* tk = ka; ka = kb; kb = tk;
    int32_t* tv = va; va = vb; vb = tv;
  }
  // segments of equal rows and their sums
  hipLaunchKernelGGL(seg_flags_kernel, dim3((unsigned)p.nblk), dim3(kThreads), 0, s, ka, L,
                     flags, counts);
  hipLaunchKernelGGL(scan_small_kernel, dim3(1), dim3(kThreads), 0, s, counts, p.nblk, total);
  hipLaunchKernelGGL(seg_starts_kernel, dim3((unsigned)p.nblk), dim3(kThreads), 0, s, flags, L,
                     counts, total, seg, n_unique);
  // at most L / (kShortMax + 1) segments are long
  const unsigned long_grid = (unsigned)std::min<int64_t>(L / (kShortMax + 1) + 1, 2048);
  const dim3 short_grid(grid_for(L, kGroups));
  if ((r & 3) == 0) {
    hipLaunchKernelGGL(seg_reduce_kernel<4>, short_grid, dim3(kThreads), 0, s, ka, va, seg,
                       n_unique, OK, r, Ly.W, Ly.use_signs, de, signs, urows, ugrad, long_list);
    hipLaunchKernelGGL(seg_reduce_long_kernel<4>, dim3(long_grid), dim3(kThreads), 0, s, va, seg,
                       long_list, OK, r, Ly.W, Ly.use_signs, de, signs, ugrad);
  } else {
    hipLaunchKernelGGL(seg_reduce_kernel<1>, short_grid, dim3(kThreads), 0, s, ka, va, seg,
                       n_unique, OK, r, Ly.W, Ly.use_signs, de, signs, urows, ugrad, long_list);
    hipLaunchKernelGGL(seg_reduce_long_kernel<1>, dim3(long_grid), dim3(kThreads), 0, s, va, seg,
                       long_list, OK, r, Ly.W, Ly.use_signs, de, signs, ugrad);
  }
  return hipGetLastError();
}

hipError_t launch_set_i64(int64_t* p, int64_t v, hipStream_t s) {
  hipLaunchKernelGGL(set_i64_kernel, dim3(1), dim3(1), 0, s, p, v);
  return hipGetLastError();
}

hipError_t launch_rms_step(const int64_t* urows, const float* ugrad, const int64_t* n_unique,
                           int64_t max_unique, int r, float* table, float* vhat, int64_t* last,
                           int64_t step, float lr, float beta2, float wd, float eps,
                           hipStream_t s) {
  hipLaunchKernelGGL(rms_step_kernel, dim3(grid_for(max_unique, kThreads / kRowLanes)), dim3(kThreads), 0,
                     s, urows, ugrad, n_unique, r, table, vhat, last, step, lr, beta2, wd, eps);
  return hipGetLastError();
}

hipError_t launch_rms_flush(int64_t R, int r, float* table, float* vhat, int64_t* last,
                            int64_t step, float lr, float beta2, float wd, hipStream_t s) {
  hipLaunchKernelGGL(rms_flush_kernel, dim3(grid_for(R, kThreads)), dim3(kThreads), 0, s, R, r,
                     table, vhat, last, step, lr, beta2, wd);
  return hipGetLastError();
}

}  // namespace pg
