// Index and gather kernels (gfx950, wave64).
//
// index:        one lane per (token, order, head): canonical IDs of the
//               n-gram, page and head hashes, row, sign words
//               (PageGram §3.1 row formula; PageGram §2.2 Engram-style rows).
// gather:       one lane per 16-byte chunk of a head row: load, dequantise
//               (NF4), apply the +-1 signs, store into the concatenated e
//               (PageGram §2.2, §3.1; Engram notes §3.2).
// index_gather: both in one kernel; a block hashes its tokens' heads into
//               LDS, then all lanes stream the rows. Lanes of a row are
//               adjacent, so each 16-head token-order is read as whole
//               contiguous rows (one 128 B segment per bf16 r=64 row, all
//               inside one K*S-row page for PageGram).
#include "common.h"

namespace pg {

// QLoRA NormalFloat levels (asymmetric standard-normal quantiles with an
// exact zero, normalised to [-1, 1]; outermost probability halfway between
// 1-1/30 and 1-1/32). Exact fp32 values.
__constant__ float kNF4[16] = {
    -0x1.0p+0f,        -0x1.647362p-1f, -0x1.0cd65cp-1f, -0x1.94653cp-2f,
    -0x1.234496p-2f,   -0x1.7a6a7ap-3f, -0x1.74f0d2p-4f, 0x0.0p+0f,
    0x1.45f602p-4f,    0x1.4995bep-3f,  0x1.f809b4p-3f,  0x1.5a066cp-2f,
    0x1.c3496ap-2f,    0x1.200f52p-1f,  0x1.722760p-1f,  0x1.0p+0f};

namespace {

constexpr int kThreads = 256;

// Elements per 16-byte input chunk and output bytes per chunk.
template <int DT> struct Chunk;
template <> struct Chunk<PG_F32> { static constexpr int epc = 4, out_bytes = 16; };
template <> struct Chunk<PG_BF16> { static constexpr int epc = 8, out_bytes = 16; };
template <> struct Chunk<PG_NF4> { static constexpr int epc = 32, out_bytes = 64; };

// Sign bits of elements [c*epc, c*epc+epc) of a head.
template <int DT>
__device__ __forceinline__ uint32_t chunk_sign_bits(const uint64_t* sw, int c) {
  constexpr int epc = Chunk<DT>::epc;
  const int e0 = c * epc;
  const uint64_t w = sw[e0 >> 6];
  return (uint32_t)(w >> (e0 & 63)) & (uint32_t)((1ull << epc) - 1);
}

// Holds one loaded chunk until it is converted and stored.
struct Raw {
  uint4 v;
  float scale;
};

template <int DT>
__device__ __forceinline__ Raw load_chunk(const uint8_t* __restrict__ table,
                                          const __half* __restrict__ scales,
                                          int64_t row, int row_bytes, int c) {
  Raw x;
  x.v = *reinterpret_cast<const uint4*>(table + row * (int64_t)row_bytes + c * 16);
  x.scale = 0.f;
  if constexpr (DT == PG_NF4) x.scale = __half2float(scales[row]);
  return x;
}

// Apply signs (and NF4 dequantisation) and store one chunk of e.
template <int DT>
__device__ __forceinline__ void store_chunk(const Raw& x, uint32_t sbits,
                                            uint8_t* __restrict__ dst,
                                            const float* cb) {
  if constexpr (DT == PG_F32) {
    uint4 o = x.v;
    o.x ^= (sbits & 1u) << 31;
    o.y ^= ((sbits >> 1) & 1u) << 31;
    o.z ^= ((sbits >> 2) & 1u) << 31;
    o.w ^= ((sbits >> 3) & 1u) << 31;
    *reinterpret_cast<uint4*>(dst) = o;
  } else if constexpr (DT == PG_BF16) {
    uint4 o = x.v;
    auto m = [&](int h) {
      return (((sbits >> (2 * h)) & 1u) << 15) | (((sbits >> (2 * h + 1)) & 1u) << 31);
    };
    o.x ^= m(0);
    o.y ^= m(1);
    o.z ^= m(2);
    o.w ^= m(3);
    *reinterpret_cast<uint4*>(dst) = o;
  } else {
    const uint32_t wds[4] = {x.v.x, x.v.y, x.v.z, x.v.w};
    uint32_t outw[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint32_t byte = (wds[b >> 2] >> (8 * (b & 3))) & 0xFFu;
      float lo = __fmul_rn(cb[byte & 15u], x.scale);
      float hi = __fmul_rn(cb[byte >> 4], x.scale);
      uint32_t blo = f32_to_bf16(lo) ^ (((sbits >> (2 * b)) & 1u) << 15);
      uint32_t bhi = f32_to_bf16(hi) ^ (((sbits >> (2 * b + 1)) & 1u) << 15);
      outw[b] = blo | (bhi << 16);
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      d4[q] = make_uint4(outw[4 * q], outw[4 * q + 1], outw[4 * q + 2], outw[4 * q + 3]);
  }
}

// The same chunk written as E4M3(e 2^s) bytes (qs = 2^s): the e value is
// the one the bf16 / fp32 path stores (sign applied; NF4 rounded to bf16
// first), scaled exactly and converted by f32x2_to_e4m3. epc bytes out.
template <int DT>
__device__ __forceinline__ void store_chunk_fp8(const Raw& x, uint32_t sbits,
                                                uint8_t* __restrict__ dst, const float* cb,
                                                float qs) {
  if constexpr (DT == PG_F32) {
    const uint32_t w[4] = {x.v.x, x.v.y, x.v.z, x.v.w};
    float v[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = __uint_as_float(w[h] ^ (((sbits >> h) & 1u) << 31)) * qs;
    *reinterpret_cast<uint32_t*>(dst) = f32x2_to_e4m3(v[0], v[1]) | (f32x2_to_e4m3(v[2], v[3]) << 16);
  } else if constexpr (DT == PG_BF16) {
    const uint32_t w[4] = {x.v.x, x.v.y, x.v.z, x.v.w};
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // elements 2q (low half) and 2q + 1 (high half) of the chunk
      const uint32_t sw = w[q] ^ (((sbits >> (2 * q)) & 1u) << 15) ^
                          (((sbits >> (2 * q + 1)) & 1u) << 31);
      const float lo = __uint_as_float(sw << 16) * qs;
      const float hi = __uint_as_float(sw & 0xFFFF0000u) * qs;
      o[q >> 1] |= f32x2_to_e4m3(lo, hi) << (16 * (q & 1));
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
  } else {
    const uint32_t wds[4] = {x.v.x, x.v.y, x.v.z, x.v.w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = 0u;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint32_t byte = (wds[b >> 2] >> (8 * (b & 3))) & 0xFFu;
      const uint32_t blo = f32_to_bf16(__fmul_rn(cb[byte & 15u], x.scale)) ^
                           (((sbits >> (2 * b)) & 1u) << 15);
      const uint32_t bhi = f32_to_bf16(__fmul_rn(cb[byte >> 4], x.scale)) ^
                           (((sbits >> (2 * b + 1)) & 1u) << 15);
      o[b >> 1] |= f32x2_to_e4m3(__uint_as_float(blo << 16) * qs,
                                 __uint_as_float(bhi << 16) * qs) << (16 * (b & 1));
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// dst[i] = E4M3(src[i] qs) for bf16 or fp32 src; a thread converts 8
// consecutive elements (16 or 32 input bytes, 8 output bytes).
__global__ __launch_bounds__(kThreads) void quantize_fp8_kernel(const void* __restrict__ src,
                                                                int dt, int64_t n, float qs,
                                                                uint8_t* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * 8;
  for (int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8; i < n; i += stride) {
    float v[8];
    const int cnt = n - i < 8 ? (int)(n - i) : 8;
    if (cnt == 8) {
      if (dt == PG_BF16) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + i);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 8; ++h)
          v[h] = __uint_as_float(((h & 1) ? (ww[h >> 1] >> 16) : (ww[h >> 1] & 0xFFFFu)) << 16);
      } else {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
      uint32_t o[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 8; h += 2)
        o[h >> 2] |= f32x2_to_e4m3(v[h] * qs, v[h + 1] * qs) << (8 * (h & 3));
      *reinterpret_cast<uint2*>(dst + i) = make_uint2(o[0], o[1]);
    } else {
      for (int h = 0; h < cnt; ++h) {
        const float x = dt == PG_BF16
                            ? bf16_to_f32(static_cast<const uint16_t*>(src)[i + h])
                            : static_cast<const float*>(src)[i + h];
        dst[i + h] = (uint8_t)(f32x2_to_e4m3(x * qs, 0.0f) & 0xFFu);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void index_kernel(
    DevLayout L, const int32_t* __restrict__ tokens, int64_t B, int64_t T,
    const int32_t* __restrict__ cmap, int64_t V, int32_t* __restrict__ canon_out,
    uint64_t* __restrict__ hash_out, int64_t* __restrict__ rows_out,
    int64_t* __restrict__ pages_out, uint64_t* __restrict__ signs_out,
    int32_t* __restrict__ status) {
  __shared__ uint64_t rc[kMaxRoles * kRoleStride];
  load_role_consts(L, rc);
  const int OK = L.O * L.K;
  const int64_t N = B * T;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= N * OK) return;
  const int64_t tok = gid / OK;
  const int rem = (int)(gid - tok * OK);
  const int i = rem / L.K;
  const int k = rem - i * L.K;
  const int64_t b = tok / T;
  const int64_t t = tok - b * T;
  const int32_t* seq = tokens + b * T;
  const int n = L.n_min + i;
  uint32_t g[kMaxOrders];
#pragma unroll
  for (int j = 0; j < kMaxOrders; ++j)
    g[j] = j < n ? canon_at(seq, t - j, cmap, V, L.pad_id) : 0;
  if (i == 0 && k == 0) {
    const int32_t tk = seq[t];
    const bool bad = tk < 0 || (int64_t)tk >= V;
    if (bad && status) atomicOr(status, 1);
    if (canon_out) canon_out[tok] = (int32_t)(bad ? L.pad_id : (uint64_t)(uint32_t)cmap[tk]);
  }
  uint64_t bh, u;
  int64_t page;
  const int64_t row = head_row(L, rc, g, i, k, &bh, &u, &page);
  rows_out[gid] = row;
  const int64_t oi = tok * L.O + i;
  if (hash_out) {
    hash_out[oi * (1 + L.K) + 1 + k] = u;
    if (k == 0) hash_out[oi * (1 + L.K)] = bh;
  }
  if (pages_out && k == 0) pages_out[oi] = page;
  for (int w = 0; w < L.W; ++w)
    signs_out[gid * L.W + w] = sign_word(L, rc, g, i, k, w);
}

// Records of the fused projection (64-element rows, one sign word). A block
// takes kRecTok tokens: their canonical IDs (and the H = n_max - 1 before
// them) are staged in LDS once, the token loads going out before the role
// constants are derived; thread (hs, token) then hashes one head slot and
// stores its record (threads loop over the (hs, token) pairs), slot-major
// so each slot's records are contiguous.
constexpr int kRecTok = 16;

// Sign bits of the fused projection's fragments: a lane of half h holds
// elements 16 st + 8 h + x (x < 8) of a 64-element row in K step st, as
// four dwords whose bits 15 and 31 are the signs of elements x = 2q and
// 2q + 1 of dword q. The word for half h puts the sign of element
// 16 st + 8 h + 2q at bit 15 - s and that of 2q + 1 at bit 31 - s, with
// s = 4 st + q, so dword q's XOR mask is (word << s) & 0x80008000.
__device__ __forceinline__ uint32_t sign_lane_word(uint64_t sw, int h) {
  // bytes 2 st + h of the word (the half's eight elements of each step)
  uint32_t x = __builtin_amdgcn_perm((uint32_t)(sw >> 32), (uint32_t)sw,
                                     h ? 0x07050301u : 0x06040200u);
  // bit unshuffle: the even bits (elements 2q) to bits 0-15, the odd ones
  // (2q + 1) to bits 16-31, each in (st, q) order
  uint32_t t = (x ^ (x >> 1)) & 0x22222222u;
  x ^= t ^ (t << 1);
  t = (x ^ (x >> 2)) & 0x0C0C0C0Cu;
  x ^= t ^ (t << 2);
  t = (x ^ (x >> 4)) & 0x00F000F0u;
  x ^= t ^ (t << 4);
  t = (x ^ (x >> 8)) & 0x0000FF00u;
  x ^= t ^ (t << 8);
  // swap the halves and reverse: (st, q) = s lands at 15 - s (odd: 31 - s)
  return __builtin_bitreverse32((x << 16) | (x >> 16));
}

__global__ __launch_bounds__(kThreads) void records_kernel(
    DevLayout L, const int32_t* __restrict__ tokens, int64_t B, int64_t T,
    const int32_t* __restrict__ cmap, int64_t V, uint4* __restrict__ rec,
    int32_t* __restrict__ status) {
  __shared__ uint64_t rc[kMaxRoles * kRoleStride];
  __shared__ uint32_t canonL[kRecTok + kMaxOrders];
  const int64_t N = B * T;
  const int64_t tok0 = (int64_t)blockIdx.x * kRecTok;
  const int tid = threadIdx.x;
  const int H = L.n_min + L.O - 2;
  const int64_t gt = tok0 - H + tid;
  const bool have = tid < kRecTok + H && gt >= 0 && gt < N;
  const int32_t tk = have ? tokens[gt] : 0;
  load_role_consts(L, rc);                      // ends with a barrier
  if (tid < kRecTok + H) {
    const bool ok = have && tk >= 0 && (int64_t)tk < V;
    canonL[tid] = ok ? (uint32_t)cmap[tk] : (uint32_t)L.pad_id;
    if (status && have && tid >= H && !ok) atomicOr(status, 1);
  }
  __syncthreads();
  for (int q = tid; q < L.O * L.K * kRecTok; q += kThreads) {
    const int hs = q / kRecTok;
    const int tl = q - hs * kRecTok;
    const int64_t tok = tok0 + tl;
    if (tok >= N) continue;
    const int i = hs / L.K;
    const int k = hs - i * L.K;
    const int64_t t = tok % T;
    const int n = L.n_min + i;
    uint32_t g[kMaxOrders];
#pragma unroll
    for (int j = 0; j < kMaxOrders; ++j)
      g[j] = j < n ? (t - j >= 0 ? canonL[H + tl - j] : (uint32_t)L.pad_id) : 0u;
    uint64_t bh, u;
    int64_t page;
    const int64_t row = head_row(L, rc, g, i, k, &bh, &u, &page);
    const uint64_t sw = sign_word(L, rc, g, i, k, 0);
    rec[hs * N + tok] = make_uint4((uint32_t)row, sign_lane_word(sw, 0), sign_lane_word(sw, 1), 0u);
  }
}

// Per-thread batch of chunk tasks kept in flight before any store.
constexpr int kBatch = 8;

template <int DT>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    int64_t n_rows, int row_bytes, int C, int OK, int W, int use_signs,
    const uint8_t* __restrict__ table, const __half* __restrict__ scales,
    const int64_t* __restrict__ rows, const uint64_t* __restrict__ signs,
    int64_t n_slots, uint8_t* __restrict__ e_out) {
  __shared__ float cb[16];
  if (threadIdx.x < 16) cb[threadIdx.x] = kNF4[threadIdx.x];
  __syncthreads();
  constexpr int OB = Chunk<DT>::out_bytes;
  const int64_t tasks = n_slots * C;
  const int64_t stride = (int64_t)gridDim.x * kThreads * kBatch;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kBatch + threadIdx.x; base < tasks;
       base += stride) {
    Raw raw[kBatch];
    int64_t slot[kBatch];
    int cc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t id = base + (int64_t)u * kThreads;
      slot[u] = -1;
      if (id < tasks) {
        slot[u] = id / C;
        cc[u] = (int)(id - slot[u] * C);
        int64_t row = rows[slot[u]];
        row = row < 0 ? 0 : (row >= n_rows ? n_rows - 1 : row);
        raw[u] = load_chunk<DT>(table, scales, row, row_bytes, cc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (slot[u] < 0) continue;
      const uint32_t sb = use_signs ? chunk_sign_bits<DT>(signs + slot[u] * W, cc[u]) : 0u;
      // e row of a token = OK head slots of C chunks each: slot-major
      // order equals the concatenation order (order outer, head inner).
      store_chunk<DT>(raw[u], sb, e_out + (slot[u] * C + cc[u]) * OB, cb);
    }
  }
}

// F8: e leaves as E4M3(e qs) bytes.
template <int DT, bool F8>
__global__ __launch_bounds__(kThreads) void index_gather_kernel(
    DevLayout L, int TB, int C, const int32_t* __restrict__ tokens, int64_t B, int64_t T,
    const int32_t* __restrict__ cmap, int64_t V, const uint8_t* __restrict__ table,
    const __half* __restrict__ scales, uint8_t* __restrict__ e_out,
    int32_t* __restrict__ status, float qs) {
  __shared__ uint64_t rc[kMaxRoles * kRoleStride];
  __shared__ int64_t rowsL[kThreads];
  __shared__ uint64_t signsL[kThreads * kMaxSignWords];
  __shared__ uint32_t canonL[kThreads + kMaxOrders];
  __shared__ float cb[16];
  const int OK = L.O * L.K;
  const int64_t N = B * T;
  const int64_t tok0 = (int64_t)blockIdx.x * TB;
  const int tid = threadIdx.x;
  // Canonical IDs of the block's tokens and the H = n_max - 1 before them,
  // loaded once per block into LDS: the token loads go out first so their
  // latency overlaps the derivation of the role constants.
  const int H = L.n_min + L.O - 2;
  const int nh = TB + H;
  int32_t tk[2];
  bool have[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + q * kThreads;
    const int64_t gt = tok0 - H + e;
    have[q] = e < nh && gt >= 0 && gt < N;
    tk[q] = have[q] ? tokens[gt] : 0;
  }
  if (threadIdx.x < 16) cb[threadIdx.x] = kNF4[threadIdx.x];
  load_role_consts(L, rc);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + q * kThreads;
    if (e >= nh) continue;
    const bool ok = have[q] && tk[q] >= 0 && (int64_t)tk[q] < V;
    canonL[e] = ok ? (uint32_t)cmap[tk[q]] : (uint32_t)L.pad_id;
    if (status && have[q] && e >= H && !ok) atomicOr(status, 1);
  }
  __syncthreads();
  if (tid < TB * OK) {
    const int tl = tid / OK;
    const int rem = tid - tl * OK;
    const int i = rem / L.K;
    const int k = rem - i * L.K;
    const int64_t tok = tok0 + tl;
    if (tok < N) {
      const int64_t t = tok % T;
      const int n = L.n_min + i;
      uint32_t g[kMaxOrders];
#pragma unroll
      for (int j = 0; j < kMaxOrders; ++j)
        g[j] = j < n ? (t - j >= 0 ? canonL[H + tl - j] : (uint32_t)L.pad_id) : 0u;
      uint64_t bh, u;
      int64_t page;
      rowsL[tid] = head_row(L, rc, g, i, k, &bh, &u, &page);
      for (int w = 0; w < L.W; ++w) signsL[tid * L.W + w] = sign_word(L, rc, g, i, k, w);
    }
  }
  __syncthreads();
  constexpr int OB = F8 ? Chunk<DT>::epc : Chunk<DT>::out_bytes;
  const int row_bytes = C * 16;
  const int64_t ntok = (N - tok0) < TB ? (N - tok0) : TB;
  const int tasks = (int)ntok * OK * C;
  uint8_t* eb = e_out + tok0 * (int64_t)OK * C * OB;
  for (int base = tid; base < tasks; base += kThreads * kBatch) {
    Raw raw[kBatch];
    int qq[kBatch], cc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int id = base + u * kThreads;
      qq[u] = -1;
      if (id < tasks) {
        qq[u] = id / C;
        cc[u] = id - qq[u] * C;
        raw[u] = load_chunk<DT>(table, scales, rowsL[qq[u]], row_bytes, cc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (qq[u] < 0) continue;
      const uint32_t sb = L.use_signs ? chunk_sign_bits<DT>(signsL + qq[u] * L.W, cc[u]) : 0u;
      if constexpr (F8)
        store_chunk_fp8<DT>(raw[u], sb, eb + ((int64_t)qq[u] * C + cc[u]) * OB, cb, qs);
      else
        store_chunk<DT>(raw[u], sb, eb + ((int64_t)qq[u] * C + cc[u]) * OB, cb);
    }
  }
}

int chunks_per_row(int32_t dt, int r) {
  return dt == PG_F32 ? r / 4 : dt == PG_BF16 ? r / 8 : r / 32;
}

}  // namespace

hipError_t launch_index(const DevLayout& L, const int32_t* tokens, int64_t B, int64_t T,
                        const int32_t* cmap, int64_t V, int32_t* canon_out,
                        uint64_t* hash_out, int64_t* rows_out, int64_t* pages_out,
                        uint64_t* signs_out, int32_t* status, hipStream_t s) {
  const int64_t total = B * T * L.O * L.K;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(index_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, L, tokens,
                     B, T, cmap, V, canon_out, hash_out, rows_out, pages_out, signs_out,
                     status);
  return hipGetLastError();
}

hipError_t launch_records(const DevLayout& L, const int32_t* tokens, int64_t B, int64_t T,
                          const int32_t* cmap, int64_t V, void* rec, int32_t* status,
                          hipStream_t s) {
  const int64_t blocks = (B * T + kRecTok - 1) / kRecTok;
  hipLaunchKernelGGL(records_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, L, tokens, B,
                     T, cmap, V, static_cast<uint4*>(rec), status);
  return hipGetLastError();
}

hipError_t launch_gather(const DevLayout& L, int32_t dt, const void* table,
                         const void* scales, const int64_t* rows, const uint64_t* signs,
                         int64_t n_tok, void* e_out, hipStream_t s) {
  const int C = chunks_per_row(dt, L.r);
  const int OK = L.O * L.K;
  const int64_t n_slots = n_tok * OK;
  const int64_t tasks = n_slots * C;
  int64_t blocks = (tasks + kThreads * kBatch - 1) / (kThreads * kBatch);
  if (blocks > 65535 * 16) blocks = 65535 * 16;
  const auto* tb = static_cast<const uint8_t*>(table);
  const auto* sc = static_cast<const __half*>(scales);
  auto* eo = static_cast<uint8_t*>(e_out);
  if (dt == PG_F32)
    hipLaunchKernelGGL(gather_kernel<PG_F32>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       L.n_rows, C * 16, C, OK, L.W, L.use_signs, tb, sc, rows, signs,
                       n_slots, eo);
  else if (dt == PG_BF16)
    hipLaunchKernelGGL(gather_kernel<PG_BF16>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       L.n_rows, C * 16, C, OK, L.W, L.use_signs, tb, sc, rows, signs,
                       n_slots, eo);
  else
    hipLaunchKernelGGL(gather_kernel<PG_NF4>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       L.n_rows, C * 16, C, OK, L.W, L.use_signs, tb, sc, rows, signs,
                       n_slots, eo);
  return hipGetLastError();
}

hipError_t launch_index_gather(const DevLayout& L, int32_t dt, const void* table,
                               const void* scales, const int32_t* tokens, int64_t B,
                               int64_t T, const int32_t* cmap, int64_t V, void* e_out,
                               int32_t* status, int e_fp8, int e_scale_exp, hipStream_t s) {
  const int C = chunks_per_row(dt, L.r);
  const int OK = L.O * L.K;
  const int TB = kThreads / OK;  // tokens per block (O*K <= 64 is validated)
  const int64_t N = B * T;
  const int64_t blocks = (N + TB - 1) / TB;
  const auto* tb = static_cast<const uint8_t*>(table);
  const auto* sc = static_cast<const __half*>(scales);
  auto* eo = static_cast<uint8_t*>(e_out);
  const float qs = ldexpf(1.0f, e_scale_exp);
#define PG_IG(DT, F8)                                                                     \
  hipLaunchKernelGGL((index_gather_kernel<DT, F8>), dim3((unsigned)blocks), dim3(kThreads), \
                     0, s, L, TB, C, tokens, B, T, cmap, V, tb, sc, eo, status, qs)
  if (e_fp8) {
    if (dt == PG_F32) PG_IG(PG_F32, true);
    else if (dt == PG_BF16) PG_IG(PG_BF16, true);
    else PG_IG(PG_NF4, true);
  } else {
    if (dt == PG_F32) PG_IG(PG_F32, false);
    else if (dt == PG_BF16) PG_IG(PG_BF16, false);
    else PG_IG(PG_NF4, false);
  }
#undef PG_IG
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* src, int32_t src_dtype, int64_t n, int scale_exp,
                               uint8_t* dst, hipStream_t s) {
  int64_t blocks = (n + kThreads * 8 - 1) / (kThreads * 8);
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, src,
                     (int)src_dtype, n, ldexpf(1.0f, scale_exp), dst);
  return hipGetLastError();
}

}  // namespace pg
