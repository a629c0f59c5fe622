// Staging of table units from a host-resident table (gfx950).
//
// Addresses are a pure function of the token IDs and are known before the
// layer runs (PageGram tech report §3.3; Engram notes §3.5), so a table kept
// in host memory can be fetched ahead: the units the step's lookups touch
// are copied once into an HBM cache, and the gather reads the cache. A page
// unit is a PageGram page (K*S rows, shared by the K heads of a token-order)
// or, for the Engram-style tables, a run of floor(4096 / row_bytes) rows of
// one per-head table starting at the table's first row; a row unit is one
// row.
//
//   clear    hash table keys <- empty
//   insert   the unit (its first row) of each lookup, by linear probing
//            (PageGram pages: one lookup per token-order: all K share one)
//   count / scan / rank
//            slot of each occupied entry = its rank in table order
//            (deterministic), unit lists by slot, the unit count
//   copy     thread per (unit, 16-byte word): its rows (and NF4 scales)
//            from the source table into cache slot s (rows s*U ..)
//   remap    cache row of each lookup = slot * U + (row - first row)
// Rows are clamped into the table, so a bad row cannot read outside it.
#include "common.h"
#include "scan.h"

namespace pg {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;                  // hash entries per thread in count / rank
constexpr uint64_t kEmpty = ~0ull;

__device__ __forceinline__ int64_t clamp_row(const DevLayout& L, int64_t row) {
  return row < 0 ? 0 : (row >= L.n_rows ? L.n_rows - 1 : row);
}

// First row of the unit holding `row` of head slot (i, k).
__device__ __forceinline__ int64_t unit_first(const DevLayout& L, int U, int64_t row, int i,
                                              int k) {
  if (U == 1) return row;
  if (L.kind == PG_PAGEGRAM) return (row / U) * U;
  const int64_t base = L.base_k[i * kMaxHeads + k];
  return base + ((row - base) / U) * U;
}

// Rows of the unit starting at f (the Engram-style tail unit of a table is
// shorter).
__device__ __forceinline__ int unit_count(const DevLayout& L, int U, int64_t f) {
  if (U == 1 || L.kind == PG_PAGEGRAM) return U;
  for (int i = 0; i < L.O; ++i)
    for (int k = 0; k < L.K; ++k) {
      const int hk = i * kMaxHeads + k;
      const int64_t end = L.base_k[hk] + (int64_t)L.Pk[hk];
      if (f >= L.base_k[hk] && f < end) return (int)(end - f < U ? end - f : U);
    }
  return 0;
}

__global__ __launch_bounds__(kThreads) void stage_clear_kernel(uint64_t* __restrict__ keys,
                                                               int64_t H) {
  for (int64_t h = (int64_t)blockIdx.x * kThreads + threadIdx.x; h < H;
       h += (int64_t)gridDim.x * kThreads)
    keys[h] = kEmpty;
}

// share: the K heads of a token-order share one unit (PageGram pages).
__global__ __launch_bounds__(kThreads) void stage_insert_kernel(
    DevLayout L, int U, int share, const int64_t* __restrict__ rows, int64_t n_look,
    uint64_t* __restrict__ keys, uint32_t mask) {
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n_look;
       q += (int64_t)gridDim.x * kThreads) {
    const int k = (int)(q % L.K);
    const int i = (int)((q / L.K) % L.O);
    if (share && k != 0) continue;
    const uint64_t f = (uint64_t)unit_first(L, U, clamp_row(L, rows[q]), i, k);
    uint32_t h = (uint32_t)(mix64(f) & mask);
    for (uint32_t probe = 0; probe <= mask; ++probe) {   // the table is never full
      const uint64_t old = atomicCAS(reinterpret_cast<unsigned long long*>(&keys[h]),
                                     (unsigned long long)kEmpty, (unsigned long long)f);
      if (old == kEmpty || old == f) break;
      h = (h + 1) & mask;
    }
  }
}

// Occupied entries of block b's kItems * kThreads range -> bcount[b].
__global__ __launch_bounds__(kThreads) void stage_count_kernel(const uint64_t* __restrict__ keys,
                                                               int64_t H,
                                                               int32_t* __restrict__ bcount) {
  __shared__ int32_t s[kThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kThreads * kItems + (int64_t)threadIdx.x * kItems;
  int32_t c = 0;
#pragma unroll
  for (int q = 0; q < kItems; ++q)
    if (base + q < H && keys[base + q] != kEmpty) ++c;
  int32_t tot;
  block_exclusive_scan<kThreads>(c, s, &tot);
  if (threadIdx.x == 0) bcount[blockIdx.x] = tot;
}

// Exclusive scan of nb block counts by one block; the total -> *n_units.
__global__ __launch_bounds__(kThreads) void stage_scan_kernel(int32_t* __restrict__ a,
                                                              int64_t nb,
                                                              int64_t* __restrict__ n_units) {
  __shared__ int32_t sh[kThreads / 64];
  const int64_t per = (nb + kThreads - 1) / kThreads;
  const int64_t lo = threadIdx.x * per, hi = lo + per < nb ? lo + per : nb;
  int32_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += a[i];
  int32_t tot;
  int32_t run = block_exclusive_scan<kThreads>(s, sh, &tot);
  if (threadIdx.x == 0) *n_units = tot;
  for (int64_t i = lo; i < hi; ++i) {
    const int32_t v = a[i];
    a[i] = run;
    run += v;
  }
}

// Slot of every occupied entry (its rank in table order) and the unit lists.
__global__ __launch_bounds__(kThreads) void stage_rank_kernel(
    DevLayout L, int U, const uint64_t* __restrict__ keys, int64_t H,
    const int32_t* __restrict__ boff, int32_t* __restrict__ ranks,
    int64_t* __restrict__ ufirst, int32_t* __restrict__ ucount) {
  __shared__ int32_t s[kThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kThreads * kItems + (int64_t)threadIdx.x * kItems;
  int32_t c = 0;
#pragma unroll
  for (int q = 0; q < kItems; ++q)
    if (base + q < H && keys[base + q] != kEmpty) ++c;
  int32_t tot;
  int32_t slot = boff[blockIdx.x] + block_exclusive_scan<kThreads>(c, s, &tot);
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int64_t h = base + q;
    if (h < H && keys[h] != kEmpty) {
      const int64_t f = (int64_t)keys[h];
      ranks[h] = slot;
      ufirst[slot] = f;
      ucount[slot] = unit_count(L, U, f);
      ++slot;
    }
  }
}

// Thread per (unit s, 16-byte word w) over the staged units: rows
// [f, f + count) of the source -> cache rows [s U, s U + count) (data rows
// are 16-byte multiples); then thread per (unit, row) for NF4 scales.
__global__ __launch_bounds__(kThreads) void stage_copy_kernel(
    const uint8_t* __restrict__ src, const __half* __restrict__ src_scales, int rb, int U,
    const int64_t* __restrict__ n_units, const int64_t* __restrict__ ufirst,
    const int32_t* __restrict__ ucount, uint8_t* __restrict__ dst,
    __half* __restrict__ dst_scales) {
  const int64_t nu = *n_units;
  const int wpu = U * rb / 16;                  // words of a full unit
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nu * wpu; g += stride) {
    const int64_t s = g / wpu;
    const int w = (int)(g - s * wpu);
    if (w < ucount[s] * rb / 16)
      reinterpret_cast<uint4*>(dst + s * U * (int64_t)rb)[w] =
          reinterpret_cast<const uint4*>(src + ufirst[s] * rb)[w];
  }
  if (src_scales)
    for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nu * U; g += stride) {
      const int64_t s = g / U;
      const int w = (int)(g - s * U);
      if (w < ucount[s]) dst_scales[s * U + w] = src_scales[ufirst[s] + w];
    }
}

__global__ __launch_bounds__(kThreads) void stage_remap_kernel(
    DevLayout L, int U, const int64_t* __restrict__ rows, int64_t n_look,
    const uint64_t* __restrict__ keys, const int32_t* __restrict__ ranks, uint32_t mask,
    int64_t* __restrict__ cache_rows) {
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n_look;
       q += (int64_t)gridDim.x * kThreads) {
    const int k = (int)(q % L.K);
    const int i = (int)((q / L.K) % L.O);
    const int64_t row = clamp_row(L, rows[q]);
    const uint64_t f = (uint64_t)unit_first(L, U, row, i, k);
    uint32_t h = (uint32_t)(mix64(f) & mask);
    int64_t slot = 0;
    for (uint32_t probe = 0; probe <= mask; ++probe) {
      const uint64_t key = keys[h];
      if (key == f) {
        slot = ranks[h];
        break;
      }
      if (key == kEmpty) break;                 // not inserted: cannot happen
      h = (h + 1) & mask;
    }
    cache_rows[q] = slot * U + (row - (int64_t)f);
  }
}

unsigned grid_for(int64_t n, int per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

StagePlan stage_plan(const DevLayout& L, int U, int share, int64_t n_tok) {
  StagePlan p{};
  p.U = U;
  p.share = share;
  p.n_look = n_tok * L.O * L.K;
  p.max_units = share ? n_tok * L.O : p.n_look;
  int64_t H = 1024;
  while (H < 2 * p.max_units) H <<= 1;
  p.H = H;
  p.nb = (H + kThreads * kItems - 1) / (kThreads * kItems);
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  int64_t off = 0;
  p.off_keys = off; off += al(H * 8);
  p.off_ranks = off; off += al(H * 4);
  p.off_bcount = off; off += al((p.nb + 1) * 4);
  p.off_ufirst = off; off += al(p.max_units * 8);
  p.off_ucount = off; off += al(p.max_units * 4);
  p.bytes = off;
  return p;
}

hipError_t launch_stage(const DevLayout& L, const StagePlan& p, int rb, const void* src,
                        const void* src_scales, const int64_t* rows, void* dst,
                        void* dst_scales, int64_t* cache_rows, int64_t* n_units,
                        int64_t* ufirst_out, void* workspace, hipStream_t s) {
  auto* ws = static_cast<uint8_t*>(workspace);
  auto* keys = reinterpret_cast<uint64_t*>(ws + p.off_keys);
  auto* ranks = reinterpret_cast<int32_t*>(ws + p.off_ranks);
  auto* bcount = reinterpret_cast<int32_t*>(ws + p.off_bcount);
  auto* ufirst = ufirst_out ? ufirst_out : reinterpret_cast<int64_t*>(ws + p.off_ufirst);
  auto* ucount = reinterpret_cast<int32_t*>(ws + p.off_ucount);
  const uint32_t mask = (uint32_t)(p.H - 1);
  hipLaunchKernelGGL(stage_clear_kernel, dim3(grid_for(p.H, kThreads)), dim3(kThreads), 0, s,
                     keys, p.H);
  hipLaunchKernelGGL(stage_insert_kernel, dim3(grid_for(p.n_look, kThreads)), dim3(kThreads), 0,
                     s, L, p.U, p.share, rows, p.n_look, keys, mask);
  hipLaunchKernelGGL(stage_count_kernel, dim3((unsigned)p.nb), dim3(kThreads), 0, s, keys, p.H,
                     bcount);
  hipLaunchKernelGGL(stage_scan_kernel, dim3(1), dim3(kThreads), 0, s, bcount, p.nb, n_units);
  hipLaunchKernelGGL(stage_rank_kernel, dim3((unsigned)p.nb), dim3(kThreads), 0, s, L, p.U, keys,
                     p.H, bcount, ranks, ufirst, ucount);
  hipLaunchKernelGGL(stage_copy_kernel,
                     dim3(grid_for(p.max_units * (int64_t)p.U * rb / 16, kThreads)),
                     dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(src), static_cast<const __half*>(src_scales),
                     rb, p.U, n_units, ufirst, ucount, static_cast<uint8_t*>(dst),
                     static_cast<__half*>(dst_scales));
  hipLaunchKernelGGL(stage_remap_kernel, dim3(grid_for(p.n_look, kThreads)), dim3(kThreads), 0,
                     s, L, p.U, rows, p.n_look, keys, ranks, mask, cache_rows);
  return hipGetLastError();
}

}  // namespace pg
