// Projection GEMMs (gfx950).
//
// Y[M x N] = E[M x K] . W[N x K]^T with bf16 inputs and fp32 accumulation on
// MFMA (v_mfma_f32_16x16x32_bf16). Both operands are K-contiguous, the layout
// the MFMA A and B fragments take directly.
//
// Main kernel (K a multiple of 32): 256 threads = 4 waves in a 2 x 2 grid,
// block tile BM x BN (256 x 192 or 256 x 256), wave tile (BM/2) x (BN/2).
// K advances BK = 64 at a time through LDS rings filled by direct
// global->LDS loads (global_load_lds_dwordx4: each lane moves 16 bytes, a
// wave writes 1 KiB of LDS per instruction), so three K tiles are in flight
// while one is multiplied and no VGPRs are spent on staging. Each stage
// buffer is its own LDS object and the loop is unrolled by the ring length so
// the compiler can tell the buffers apart; the ring is synchronised with
// counted vmcnt waits and a bare barrier (a __syncthreads() would drain every
// outstanding load). Within a 64-byte LDS row the four 16-byte K chunks are
// XOR-swizzled by (row >> 1) & 3, so the 16 rows a fragment read touches fall
// in distinct banks. Rows past M or N are clamped in-bounds for the loads and
// never stored.
//
// Blocks are renumbered so that each XCD (blocks are dealt round-robin to the
// 8 XCDs) runs a contiguous range of M-major tiles: the N tiles of one E tile
// run together on one XCD and share that E tile and W through its L2.
//
// Fallback kernel (K a multiple of 8): 128 x 128 tile, BK = 64, register-
// staged double buffer; scalar gate only.
//
// Epilogues: the scalar gate (PageGram §3.1: out = x + g W_V e) and pass 1 of
// the Engram fusion (Engram notes §3.3-3.4): v = W_V e is stored in bf16 and,
// per token and 128-column block, the partial sums RMSNorm and the context
// gate need (sum v^2; per branch sum k^2, sum gamma_h gamma_k h k, sum h^2)
// go to the workspace, so k is never stored.
//
// fp32: a plain LDS-tiled FMA GEMM for fp32 tables (tiny workloads).
#include "common.h"

namespace pg {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kThreads = 256;
constexpr int kColBlock = 256;   // Engram partial-sum column block
#ifndef PIPE_BK
#define PIPE_BK 64
#endif
#ifndef PIPE_STAGES
#define PIPE_STAGES 2
#endif

enum { EPI_SCALAR = 0, EPI_ENGRAM = 1 };

struct EpiArgs {
  // scalar gate
  float g;
  const uint16_t* resid;   // [M][N] or NULL
  uint16_t* out;           // [M][N]
  // Engram pass 1
  int d;
  int n_cb;                // d / 256 column blocks per segment
  const uint16_t* h;       // [Mbr][M][d]
  uint16_t* v;             // [M][d]
  float* part_v;           // [n_cb][M]
  float* part_k;           // [Mbr][3][n_cb][M]
  const float* gamma_h;
  const float* gamma_k;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// s_waitcnt with only a vmcnt limit (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One direct global->LDS load: each lane moves 16 bytes from `src`; the wave
// writes 1 KiB at LDS byte address `lds` (wave-uniform, passed in M0) +
// 16 * lane. Issued as inline asm without a memory clobber, so the compiler's
// wait-count pass neither tracks it nor waits for it before LDS reads (its
// LDS-DMA tracking would otherwise wait for every outstanding load). The ring
// orders it explicitly: counted vmcnt waits, then a barrier fenced on both
// sides by compiler-only memory barriers; volatile asm keeps its order.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

__device__ __forceinline__ int64_t remap_block(int64_t bid, int64_t total) {
  const int64_t per = total / 8;
  if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
  return bid;
}

// Tile of a (renumbered) block id: groups of kGroupM M tiles, each group
// walked N-major, so the blocks running together on an XCD share a few E
// tiles and a few W tiles instead of one E tile and all of W.
constexpr int kGroupM = 8;
__device__ __forceinline__ void block_tile(int64_t id, int64_t nbm, int64_t nbn, int64_t* bm,
                                           int64_t* bn) {
  const int64_t per_group = (int64_t)kGroupM * nbn;
  const int64_t g = id / per_group;
  const int64_t local = id - g * per_group;
  const int64_t rows = nbm - g * kGroupM < kGroupM ? nbm - g * kGroupM : kGroupM;
  *bn = local / rows;
  *bm = g * kGroupM + (local - *bn * rows);
}

// Scalar-gate epilogue for a wave's FM x FN accumulator tiles.
template <int FM, int FN>
__device__ __forceinline__ void epi_scalar(const f32x4_t (&acc)[FM][FN], int64_t row0,
                                           int col0, int lane, int64_t M, int N,
                                           const EpiArgs& ep) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = row0 + i * 16 + 4 * (lane >> 4) + q;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 16 + (lane & 15);
        if (col >= N) continue;
        const int64_t o = row * N + col;
        const float x = ep.resid ? bf16_to_f32(ep.resid[o]) : 0.f;
        ep.out[o] = f32_to_bf16(x + ep.g * acc[i][j][q]);
      }
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel

// LDS bytes of the K ring and of the epilogue's staging tile.
template <int BM, int BN, int BK, int S>
struct PipeCfg {
  // E ring of S buffers (E tiles S-1 stages ahead) and W ring of 2 buffers
  // (one stage ahead): E comes from further away (MALL/HBM) than W (L2).
  static constexpr int kABytes = BM * BK * 2;
  static constexpr int kBBytes = BN * BK * 2;
  static constexpr int kBOffset = S * kABytes;
  static constexpr int kRingBytes = S * kABytes + 2 * kBBytes;
  static constexpr int kPad = 4;                 // floats of row padding
  static constexpr int kRowStride = BN + kPad;   // staged accumulator row (floats)
  // rows of the block tile staged per epilogue pass: as many wave rows
  // (BM/2) as fit beside nothing else (the ring is dead by then)
  static constexpr int kPassRows =
      (BM / 2) * kRowStride * 4 <= kRingBytes ? BM / 2 : BM / 4;
  static constexpr int kStageTileBytes = kPassRows * kRowStride * 4;
  static constexpr int kLdsBytes = kRingBytes > kStageTileBytes ? kRingBytes : kStageTileBytes;
};

template <int BM, int BN, int BK, int S, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_pipe_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bw, int64_t M, int N,
    int K, EpiArgs ep) {
  using Cfg = PipeCfg<BM, BN, BK, S>;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int LPR = BK / 8;                  // 16-byte chunks (lanes) per row
  constexpr int RPI = 64 / LPR;                // rows per DMA instruction
  constexpr int ROWS_PER_LINE = 64 / BK;       // rows per 128-byte LDS line
  constexpr int A_DMA = BM / RPI / 4;          // DMA instructions per wave per stage
  constexpr int B_DMA = BN / RPI / 4;
  constexpr int L = A_DMA + B_DMA;
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(BM % (4 * RPI) == 0 && BN % (4 * RPI) == 0, "tile split");
  static_assert(S == 2 || S == 3, "E ring of 2 or 3 buffers");
  static_assert(L + A_DMA < 64, "vmcnt range");
  static_assert(Cfg::kLdsBytes <= 160 * 1024, "LDS");
  static_assert(EPI != EPI_ENGRAM || BN == kColBlock, "an Engram tile is one column block");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t nbm = (M + BM - 1) / BM;
  const int64_t nbn = (N + BN - 1) / BN;
  int64_t bm, bn;
  block_tile(remap_block(blockIdx.x, nbm * nbn), nbm, nbn, &bm, &bn);
  const int64_t m0 = bm * BM;
  const int n0 = (int)(bn * BN);

  // The epilogue's bf16 input tile -- the residual x (scalar gate, N a
  // multiple of 8) or h of this branch (Engram k tiles) -- is fetched at the
  // start so its latency overlaps the first K tiles. Chunk q of this thread is
  // epilogue item tid + 256 q (row-major 8-column chunks of the block tile).
  constexpr int CPR = BN / 8;                   // 8-column chunks per row
  constexpr int PCH = BM * BN / 8 / kThreads;
  uint4 pre[PCH];
  bool pre_ok;
  const uint16_t* pre_src;
  int64_t pre_ld;
  int pre_c0;
  if constexpr (EPI == EPI_SCALAR) {
    pre_ok = ep.resid != nullptr && (N & 7) == 0;
    pre_src = ep.resid;
    pre_ld = N;
    pre_c0 = n0;
  } else {
    const int seg = n0 / ep.d;
    pre_ok = seg > 0;
    pre_src = seg > 0 ? ep.h + (int64_t)(seg - 1) * M * ep.d : ep.h;
    pre_ld = ep.d;
    pre_c0 = n0 - seg * ep.d;
  }
  // Chunks fetched at the start; the rest are fetched when the epilogue
  // begins (the 256 x 256 tile has no registers for all of them in the loop).
  constexpr int PEARLY = BM * BN > 256 * 192 ? PCH / 2 : PCH;
  auto fetch_pre = [&](int q) {
    const int idx = tid + q * kThreads;
    const int64_t row = m0 + idx / CPR;
    const int cc = (idx % CPR) * 8;
    pre[q] = make_uint4(0, 0, 0, 0);
    if (pre_ok && row < M && n0 + cc < N)
      pre[q] = *reinterpret_cast<const uint4*>(pre_src + row * pre_ld + pre_c0 + cc);
  };
#pragma unroll
  for (int q = 0; q < PEARLY; ++q) fetch_pre(q);

  // Swizzle of the 16-byte chunk position within a row: rows sharing a
  // 128-byte line, and the next lines, rotate their chunks.
  auto swz = [](int r) { return (r / ROWS_PER_LINE) & (LPR - 1); };

  // DMA: lane covers row lane / LPR of an RPI-row slab and LDS chunk position
  // lane % LPR, loading the logical chunk pos ^ swz(row).
  const int dr = lane / LPR;
  const int dpos = lane % LPR;
  const uint16_t* a_src[A_DMA];
  const uint16_t* b_src[B_DMA];
#pragma unroll
  for (int j = 0; j < A_DMA; ++j) {
    const int r = (wave * A_DMA + j) * RPI + dr;
    int64_t gm = m0 + r;
    gm = gm < M ? gm : M - 1;
    a_src[j] = A + gm * (int64_t)K + ((dpos ^ swz(r)) * 8);
  }
#pragma unroll
  for (int j = 0; j < B_DMA; ++j) {
    const int r = (wave * B_DMA + j) * RPI + dr;
    int gn = n0 + r;
    gn = gn < N ? gn : N - 1;
    b_src[j] = Bw + (int64_t)gn * K + ((dpos ^ swz(r)) * 8);
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue_a = [&](int kt) {
    const uint32_t la = lds0 + (kt % S) * Cfg::kABytes + wave * A_DMA * 1024;
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) dma16(a_src[j] + kt * BK, la + j * 1024);
  };
  auto issue_b = [&](int kt) {
    const uint32_t lb = lds0 + Cfg::kBOffset + (kt & 1) * Cfg::kBBytes + wave * B_DMA * 1024;
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) dma16(b_src[j] + kt * BK, lb + j * 1024);
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragment read: lane reads row (lane & 15) of a 16-row tile, logical chunk
  // ks * 4 + (lane >> 4), stored at that chunk ^ swz(row).
  const int fr = lane & 15;
  auto compute = [&](int kt) {
    const uint16_t* sa = reinterpret_cast<const uint16_t*>(smem + (kt % S) * Cfg::kABytes);
    const uint16_t* sb =
        reinterpret_cast<const uint16_t*>(smem + Cfg::kBOffset + (kt & 1) * Cfg::kBBytes);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int pos = ((ks * 4 + (lane >> 4)) ^ swz(fr)) * 8;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
            &sa[(wm * WTM + i * 16 + fr) * BK + pos]));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(
            &sb[(wn * WTN + j * 16 + fr) * BK + pos]));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  const int KT = K / BK;
  // Issue order: W(kt+1) then E(kt+S-1) each step, after W(0), E(0..S-2).
  // The wait at step kt needs E(kt) and W(kt); with S = 3 the only load
  // issued after W(kt) is E(kt+1), which may stay in flight.
  issue_b(0);
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT) issue_a(s);
  for (int kt = 0; kt < KT; ++kt) {
    if (S == 3 && kt + 1 < KT)
      wait_vmcnt<(S == 3 ? A_DMA : 0)>();
    else
      wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // buffers refilled here were last read by compute(kt - 1)
    if (kt + 1 < KT) issue_b(kt + 1);
    if (kt + S - 1 < KT) issue_a(kt + S - 1);
    compute(kt);
  }

  // Epilogue: stage the accumulators through LDS, kPassRows rows at a time,
  // so global traffic is 16-byte loads and stores along rows.
  float* tile = reinterpret_cast<float*>(smem);
  constexpr int R = Cfg::kPassRows;
  constexpr int RS = Cfg::kRowStride;
  constexpr int ITEMS = R * CPR / kThreads;     // items per thread per pass
  static_assert(R * CPR % kThreads == 0, "epilogue items");
#pragma unroll
  for (int q = PEARLY; q < PCH; ++q) fetch_pre(q);
#pragma unroll
  for (int p = 0; p < BM / R; ++p) {
    asm volatile("" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rl = wm * WTM + i * 16 + 4 * (lane >> 4) + q - p * R;
        if (rl < 0 || rl >= R) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          tile[rl * RS + wn * WTN + j * 16 + (lane & 15)] = acc[i][j][q];
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * kThreads;
      const int rl = idx / CPR;
      const int c8 = (idx - rl * CPR) * 8;
      const int64_t row = m0 + p * R + rl;
      const int col = n0 + c8;
      const float4 lo = *reinterpret_cast<const float4*>(&tile[rl * RS + c8]);
      const float4 hi = *reinterpret_cast<const float4*>(&tile[rl * RS + c8 + 4]);
      const float y[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float xin[8];
      {
        const uint4 pr = pre[p * ITEMS + it];
        const uint32_t pw[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xin[2 * u] = bf16_to_f32((uint16_t)(pw[u] & 0xFFFFu));
          xin[2 * u + 1] = bf16_to_f32((uint16_t)(pw[u] >> 16));
        }
      }
      if constexpr (EPI == EPI_SCALAR) {
        if (row >= M) continue;
        if (pre_ok || (ep.resid == nullptr && col + 8 <= N && (N & 7) == 0)) {
          if (col >= N) continue;
          uint32_t ow[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            ow[u] = (uint32_t)f32_to_bf16(xin[2 * u] + ep.g * y[2 * u]) |
                    ((uint32_t)f32_to_bf16(xin[2 * u + 1] + ep.g * y[2 * u + 1]) << 16);
          *reinterpret_cast<uint4*>(ep.out + row * N + col) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        } else {
          for (int u = 0; u < 8 && col + u < N; ++u) {
            const int64_t o = row * N + col + u;
            const float x = ep.resid ? bf16_to_f32(ep.resid[o]) : 0.f;
            ep.out[o] = f32_to_bf16(x + ep.g * y[u]);
          }
        }
      } else {
        // Engram pass 1: the block's 256 columns are one partial-sum column
        // block of one segment (BN = 256 divides d); the 32 consecutive lanes
        // of a row hold it.
        const bool live = row < M;
        const int seg = col / ep.d;
        const int c = col - seg * ep.d;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
        if (seg == 0) {
          uint32_t vw[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            vw[u] = (uint32_t)f32_to_bf16(y[2 * u]) | ((uint32_t)f32_to_bf16(y[2 * u + 1]) << 16);
          if (live)
            *reinterpret_cast<uint4*>(ep.v + row * ep.d + c) = make_uint4(vw[0], vw[1], vw[2], vw[3]);
#pragma unroll
          for (int u = 0; u < 8; ++u) s0 += y[u] * y[u];
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            s0 += y[u] * y[u];
            s1 += ep.gamma_h[c + u] * ep.gamma_k[c + u] * xin[u] * y[u];
            s2 += xin[u] * xin[u];
          }
        }
#pragma unroll
        for (int sh = 1; sh < CPR; sh <<= 1) {
          s0 += __shfl_xor(s0, sh, 64);
          s1 += __shfl_xor(s1, sh, 64);
          s2 += __shfl_xor(s2, sh, 64);
        }
        if (live && (lane % CPR) == 0) {
          const int cb = c / kColBlock;
          if (seg == 0) {
            ep.part_v[(int64_t)cb * M + row] = s0;
          } else {
            float* pk = ep.part_k + (int64_t)(seg - 1) * 3 * ep.n_cb * M;
            pk[((int64_t)0 * ep.n_cb + cb) * M + row] = s0;
            pk[((int64_t)1 * ep.n_cb + cb) * M + row] = s1;
            pk[((int64_t)2 * ep.n_cb + cb) * M + row] = s2;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fallback kernel (K % 8 == 0), scalar gate

constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;   // padded LDS row (elements)

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bw, int64_t M, int N,
    int K, EpiArgs ep) {
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_IT = BM * kBK / 8 / kThreads;
  constexpr int B_IT = BN * kBK / 8 / kThreads;
  static_assert(A_IT >= 1 && B_IT >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kLDK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t nbm = (M + BM - 1) / BM;
  const int64_t nbn = (N + BN - 1) / BN;
  const int64_t bid = remap_block(blockIdx.x, nbm * nbn);
  const int64_t bm = bid / nbn;
  const int64_t bn = bid - bm * nbn;
  const int64_t m0 = bm * BM;
  const int n0 = (int)(bn * BN);

  const int lc = tid & 7;    // 16-byte chunk within a 64-element K row
  const int lr = tid >> 3;   // row 0..31, plus 32 per iteration

  uint4 ra[A_IT], rb[B_IT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int64_t gm = m0 + lr + 32 * it;
      const int kk = k0 + lc * 8;
      ra[it] = (gm < M && kk < K)
                   ? *reinterpret_cast<const uint4*>(A + gm * (int64_t)K + kk)
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < B_IT; ++it) {
      const int gn = n0 + lr + 32 * it;
      const int kk = k0 + lc * 8;
      rb[it] = (gn < N && kk < K)
                   ? *reinterpret_cast<const uint4*>(Bw + (int64_t)gn * K + kk)
                   : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it)
      *reinterpret_cast<uint4*>(&As[buf][(lr + 32 * it) * kLDK + lc * 8]) = ra[it];
#pragma unroll
    for (int it = 0; it < B_IT; ++it)
      *reinterpret_cast<uint4*>(&Bs[buf][(lr + 32 * it) * kLDK + lc * 8]) = rb[it];
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = (K + kBK - 1) / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8_t af[FM], bf[FN];
      const int koff = ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
            &As[cur][(wm * WTM + i * 16 + (lane & 15)) * kLDK + koff]));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[j] = as_bf16x8(*reinterpret_cast<const uint4*>(
            &Bs[cur][(wn * WTN + j * 16 + (lane & 15)) * kLDK + koff]));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }
  epi_scalar<FM, FN>(acc, m0 + wm * WTM, n0 + wn * WTN, lane, M, N, ep);
}

// fp32: 64 x 64 tile, BK = 16, each thread a 4 x 4 block of outputs.
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ Bw, int64_t M, int N, int K,
    float g, const float* __restrict__ resid, float* __restrict__ out) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[BK][BN + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int e = tid; e < BM * BK; e += kThreads) {
      const int r = e / BK, kk = e % BK;
      const int64_t gm = m0 + r;
      As[kk][r] = (gm < M && k0 + kk < K) ? A[gm * K + k0 + kk] : 0.f;
      const int gn = n0 + r;
      Bs[kk][r] = (gn < N && k0 + kk < K) ? Bw[(int64_t)gn * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      const int64_t o = row * N + col;
      out[o] = (resid ? resid[o] : 0.f) + g * acc[i][j];
    }
  }
}

template <int BM, int BN, int EPI>
hipError_t launch_pipe(const void* e, int64_t M, int N, int K, const void* W,
                       const EpiArgs& ep, hipStream_t s) {
  constexpr int BK = PIPE_BK, S = PIPE_STAGES;
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, BK, S, EPI>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(e),
                     static_cast<const uint16_t*>(W), M, N, K, ep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project_scalar(int32_t dtype, const void* e, int64_t N, int64_t E,
                                 const void* W, int64_t d, float g, const void* resid,
                                 void* out, hipStream_t s) {
  if (dtype == PG_F32) {
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)((d + 63) / 64));
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(e), static_cast<const float*>(W), N, (int)d,
                       (int)E, g, static_cast<const float*>(resid), static_cast<float*>(out));
    return hipGetLastError();
  }
  EpiArgs ep{};
  ep.g = g;
  ep.resid = static_cast<const uint16_t*>(resid);
  ep.out = static_cast<uint16_t*>(out);
  if (E % PIPE_BK == 0) {
    // Pick the N tile by rounds of 256 concurrent blocks times block work.
    auto cost = [&](int64_t bn) {
      const int64_t blocks = ((N + 255) / 256) * ((d + bn - 1) / bn);
      return ((blocks + 255) / 256) * bn;
    };
    if (cost(192) < cost(256))
      return launch_pipe<256, 192, EPI_SCALAR>(e, N, (int)d, (int)E, W, ep, s);
    return launch_pipe<256, 256, EPI_SCALAR>(e, N, (int)d, (int)E, W, ep, s);
  }
  constexpr int BM = 128, BN = 128;
  const int64_t blocks = ((N + BM - 1) / BM) * ((d + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(e), static_cast<const uint16_t*>(W), N,
                     (int)d, (int)E, ep);
  return hipGetLastError();
}

// Engram pass 1 (E % 32 == 0 and d % 256 == 0, checked by the caller).
hipError_t launch_engram_pass1(const void* e, int64_t N, int64_t E, const void* W,
                               int64_t d, int64_t Mbr, const void* h,
                               const float* gamma_h, const float* gamma_k, uint16_t* v,
                               float* part_v, float* part_k, hipStream_t s) {
  EpiArgs ep{};
  ep.d = (int)d;
  ep.n_cb = (int)(d / kColBlock);
  ep.h = static_cast<const uint16_t*>(h);
  ep.v = v;
  ep.part_v = part_v;
  ep.part_k = part_k;
  ep.gamma_h = gamma_h;
  ep.gamma_k = gamma_k;
  return launch_pipe<256, 256, EPI_ENGRAM>(e, N, (int)((1 + Mbr) * d), (int)E, W, ep, s);
}

}  // namespace pg
