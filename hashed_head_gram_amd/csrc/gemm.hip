// Projection GEMMs (gfx950).
//
// Y[M x N] = E[M x K] . W[N x K]^T with bf16 inputs and fp32 accumulation on
// the matrix cores. Both operands are K-contiguous, the layout the MFMA A and
// B fragments take directly.
//
// Main kernel (K a multiple of 64): 512 threads = 8 waves, two per SIMD, so
// one wave's matrix work covers the other's barrier and LDS waits; block
// tile BM x BN (256 x 192 in a 4 x 2 wave grid, or 256 x 256 in 2 x 4),
// wave tile 64 x 96 or 128 x 64 made of 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16 (measured faster in these kernels than 16 x 16 x 32,
// although with register operands alone the 16 x 16 form issues a little
// faster). K advances 64 at a
// time through two-buffer LDS rings for the E and W tiles, filled by direct
// global->LDS loads (global_load_lds_dwordx4: a lane moves 16 bytes, a wave
// writes 1 KiB of LDS per instruction; the address is an SGPR base plus a
// per-lane offset), so no VGPRs are spent on staging. A stage's four K steps
// interleave: the LDS fragment reads of step s+1 go out between the MFMAs of
// step s; the next stage's loads all go out at the top of the stage. The
// W fragment is the MFMA's A operand, so each lane's accumulators are runs
// of four consecutive output columns of one token row. The ring is
// synchronised with counted vmcnt waits and a bare barrier (a
// __syncthreads() would drain every outstanding load). The four 16-byte K
// chunks of a row are XOR-swizzled per 256-byte line so a fragment read is
// free of bank conflicts. Rows past M or N are clamped in-bounds for the
// loads and never stored.
//
// Blocks are renumbered so that each XCD (blocks are dealt round-robin to the
// 8 XCDs) runs a contiguous range of tiles, walked in groups of 8 M tiles
// N-major: concurrently running tiles share their E and W panels in one L2.
//
// Epilogue: the accumulators are staged through LDS a pass of rows at a
// time (one 16-byte LDS write per four columns) and leave as 16-byte row
// stores; passes synchronise on LDS only (the stores are never waited for);
// the bf16 residual tile is fetched once before the first store; bf16
// packing is one v_cvt_pk_bf16_f32 per pair. Two epilogues: the scalar gate
// (PageGram §3.1: out = x + g W_V e) and fp32 output (the backward's GEMMs).
// Pass 1 of the Engram fusion runs on the slot-ring kernel of gemm_slots.hip.
//
// Fallback kernel (K a multiple of 8): 128 x 128 tile, BK = 64, register-
// staged double buffer; scalar gate only.
//
// fp32: a plain LDS-tiled FMA GEMM for fp32 tables (tiny workloads).
#include <type_traits>

#include "common.h"

namespace pg {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));   // 32 FP8 values
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kThreads = 256;
constexpr int kPipeBK = 64;      // K stage of the pipelined kernel (bf16 elements)
constexpr int kPipeBK8 = 128;    // the same 128 bytes per row in FP8 elements
constexpr int kPipeStages = 2;   // its LDS ring

enum { EPI_SCALAR = 0, EPI_F32 = 2 };

struct EpiArgs {
  // scalar gate
  float g;
  const uint16_t* resid;   // [M][N] or NULL
  uint16_t* out;           // [M][N]
  // fp32 output (g * acc): out_f32[row * ldo + col]; with split K, block
  // column blockIdx.y covers K range [y K, (y+1) K) of the operands and
  // writes its partial product at out_f32 + y * M * ldo
  float* out_f32;
  int64_t ldo;
  // operand row strides in elements (0: K)
  int lda, ldb;
  // FP8 operands: E8M0 scales of the MFMA's A (W) and B (e) operands,
  // 127 - s for an operand stored as E4M3(v 2^s)
  int f8_sa, f8_sb;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even) in one instruction
// (v_cvt_pk_bf16_f32); `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

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
// The address is a wave-uniform base (SGPR pair) plus a per-lane 32-bit
// byte offset, so a stage's loads hold one VGPR per lane instead of a 64-bit
// pointer per instruction.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds));
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
        ep.out[o] = (uint16_t)pack_bf16x2(x + ep.g * acc[i][j][q], 0.f);
      }
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel

// LDS bytes of the K ring and of the epilogue's staging tile; BKB is the
// bytes of one row's K stage.
template <int BM, int BN, int BKB, int S>
struct PipeCfg {
  // rings of S buffers for the E and the W tiles (S - 1 stages in flight)
  static constexpr int kABytes = BM * BKB;
  static constexpr int kBBytes = BN * BKB;
  static constexpr int kBOffset = S * kABytes;
  static constexpr int kRingBytes = S * (kABytes + kBBytes);
  static constexpr int kPad = 4;                 // floats of row padding
  static constexpr int kRowStride = BN + kPad;   // staged accumulator row (floats)
  // rows of the block tile staged per epilogue pass: half the tile if it
  // fits in the ring's bytes (the ring is dead by then), else a quarter
  static constexpr int kPassRows =
      (BM / 2) * kRowStride * 4 <= kRingBytes ? BM / 2 : BM / 4;
  static constexpr int kStageTileBytes = kPassRows * kRowStride * 4;
  static constexpr int kLdsBytes = kRingBytes > kStageTileBytes ? kRingBytes : kStageTileBytes;
};

// Gathered projection (pg_forward with a bf16 table of 64-element rows):
// the E tile of K stage kt is head slot kt of the tile's tokens, so its rows
// are table rows, loaded straight into the ring from the table by the
// per-(head slot, token) records records_kernel wrote. The records of a
// head slot are DMA'd into LDS three stages ahead, the rows of a stage read
// from them into registers one stage before the stage's DMA, and the +-1
// signs applied to the E fragments after the LDS read (a shift, an AND and
// an XOR per dword, the sign bits being pre-arranged in fragment order).
struct GatherArgs {
  const uint8_t* table;        // [R][64] bf16 rows (R * 128 bytes < 2^32)
  const uint8_t* rec;          // [K / 64][M] records {row, sign words of the two
                               // lane halves, 0}
};

// WGM x WGN waves (64 WGM WGN threads): 2 x 2 puts one wave on each SIMD;
// 2 x 4 and 4 x 2 put two, so one wave's matrix work covers the other's
// barrier and LDS waits. F8: E4M3 operands (BK = 128 K elements per stage)
// on v_mfma_scale_f32_32x32x64_f8f6f4, whose E8M0 operand scales undo the
// operands' power-of-two scaling; otherwise bf16 (BK = 64) on
// v_mfma_f32_32x32x16_bf16. Either way a row's K stage is 128 bytes.
template <int BM, int BN, int BK, int S, int EPI, int WGM, int WGN, bool F8, bool GATHER>
__device__ __forceinline__ void pipe_body(const uint8_t* __restrict__ A,
                                          const uint8_t* __restrict__ Bw, int64_t M, int N,
                                          int K, const EpiArgs& ep, const GatherArgs& ga) {
  constexpr int EB = F8 ? 1 : 2;                // operand element bytes
  constexpr int BKB = BK * EB;                  // bytes of a row's K stage
  using Cfg = PipeCfg<BM, BN, BKB, S>;
  constexpr int NW = WGM * WGN;                 // waves
  constexpr int NT = 64 * NW;                   // threads
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;   // 32 x 32 MFMA tiles per wave
  constexpr int LPR = BKB / 16;                // 16-byte chunks (lanes) per row
  constexpr int RPI = 64 / LPR;                // rows per DMA instruction
  constexpr int ROWS_PER_LINE = 256 / BKB;     // rows per 256-byte LDS line
  constexpr int A_DMA = BM / RPI / NW;         // DMA instructions per wave per stage
  constexpr int B_DMA = BN / RPI / NW;
  constexpr int L = A_DMA + B_DMA;
  static_assert(BKB == 64 || BKB == 128, "K stage of 64 or 128 bytes");
  static_assert(S >= 2 && S <= 4, "ring of 2 to 4 stages");
  static_assert(2 * L < 64, "vmcnt range");
  static_assert(BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "tile split");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "whole 32 x 32 MFMA tiles per wave");
  static_assert(L < 64, "vmcnt range");
  static_assert(Cfg::kLdsBytes <= 160 * 1024, "LDS");
  static_assert(!GATHER || (!F8 && BKB == 128 && EPI == EPI_SCALAR && S == 2 && NT >= BM),
                "fused gather: bf16 64-element rows, scalar gate");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::kLdsBytes];
  // fused gather: the records of four head slots (rows and sign words of
  // the tile's tokens)
  __shared__ __attribute__((aligned(16))) uint4 recL[GATHER ? 4 : 1][GATHER ? BM : 1];

  const int64_t lda = ep.lda ? ep.lda : K;
  const int64_t ldb = ep.ldb ? ep.ldb : K;
  if constexpr (EPI == EPI_F32) {
    A += (int64_t)blockIdx.y * K * EB;
    Bw += (int64_t)blockIdx.y * K * EB;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WGN, wn = wave % WGN;

  const int64_t nbm = (M + BM - 1) / BM;
  const int64_t nbn = (N + BN - 1) / BN;
  int64_t bm, bn;
  block_tile(remap_block(blockIdx.x, nbm * nbn), nbm, nbn, &bm, &bn);
  const int64_t m0 = bm * BM;
  const int n0 = (int)(bn * BN);

  // The epilogue's bf16 input tile -- the residual x (scalar gate, N a
  // multiple of 8) or h of this branch (Engram k tiles). Chunk q of this
  // thread is epilogue item tid + 256 q (row-major 8-column chunks of the
  // block tile); each epilogue pass fetches its own chunks before staging
  // the accumulators, so the loads overlap the LDS round trip and the main
  // loop keeps its registers for the fragment pipeline.
  constexpr int CPR = BN / 8;                   // 8-column chunks per row
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
    pre_ok = false;
    pre_src = nullptr;
    pre_ld = 0;
    pre_c0 = 0;
  }

  // Swizzle of the 16-byte chunk position within a row. gfx950's LDS serves
  // 256 bytes per clock, so the 16 lanes that a 16-byte read serves together
  // must hit 16 distinct 16-byte slots of a 256-byte line: the rows sharing
  // a line differ in their half, and consecutive lines rotate the chunks.
  auto swz = [](int r) { return (r / ROWS_PER_LINE) & (LPR - 1); };

  // DMA: lane covers row lane / LPR of an RPI-row slab and LDS chunk position
  // lane % LPR, loading the logical chunk pos ^ swz(row).
  // Each instruction covers the RPI-row group g = wave * X_DMA + j; the
  // group's first row (clamped to the last valid row) is the scalar base and
  // rows past the matrix repeat its last row (never stored).
  const int dr = lane / LPR;
  const int dpos = lane % LPR;
  // A group's first row r0 is a multiple of RPI (and the tile origin a
  // multiple of 16 rows), so swz(r0 + dr) = swz(r0) ^ swz(dr) with swz(r0)
  // fixed by the group index.
  const uint32_t chunk_b = (uint32_t)((dpos ^ swz(dr)) * 16);
  const uint32_t lds0 = lds_addr(smem);
  auto issue_rows = [&](const uint8_t* mat, int64_t ld, int64_t rows, int64_t r0, int grp,
                        int kt, uint32_t lds) {
    int64_t rb = r0 < rows ? r0 : rows - 1;
    const int lim = (int)(rows - 1 - rb);
    const int rr = dr < lim ? dr : lim;
    dma16(mat + (rb * ld + (int64_t)kt * BK) * EB,
          (uint32_t)(rr * ld * EB) + (chunk_b ^ (uint32_t)(swz(grp * RPI) * 16)), lds);
  };
  // fused gather: the lane's table rows of the next stage to load (head
  // slot hs, token rows grp * RPI + dr), read from the records one stage
  // before their DMA so the DMA waits on no LDS read
  uint32_t nrow[GATHER ? A_DMA : 1];
  auto read_rows = [&](int hs) {
    if constexpr (GATHER) {
#pragma unroll
      for (int j = 0; j < A_DMA; ++j) nrow[j] = recL[hs % 4][(wave * A_DMA + j) * RPI + dr].x;
    }
  };
  auto issue_a = [&](int kt) {
    const uint32_t la = lds0 + (kt % S) * Cfg::kABytes + wave * A_DMA * 1024;
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
      if constexpr (GATHER) {
        const int grp = wave * A_DMA + j;
        dma16(ga.table, nrow[j] * 128u + (chunk_b ^ (uint32_t)(swz(grp * RPI) * 16)),
              la + j * 1024);
      } else {
        issue_rows(A, lda, M, m0 + (wave * A_DMA + j) * RPI, wave * A_DMA + j, kt,
                   la + j * 1024);
      }
    }
  };
  auto issue_b = [&](int kt) {
    const uint32_t lb = lds0 + Cfg::kBOffset + (kt % S) * Cfg::kBBytes + wave * B_DMA * 1024;
#pragma unroll
    for (int j = 0; j < B_DMA; ++j)
      issue_rows(Bw, ldb, N, n0 + (wave * B_DMA + j) * RPI, wave * B_DMA + j, kt, lb + j * 1024);
  };
  // fused gather: DMA of head slot hs's records for the tile's tokens into
  // buffer hs % 4, by the first BM / 64 waves (tokens past M repeat the
  // last token's record)
  auto issue_rec = [&](int hs) {
    if constexpr (GATHER) {
      if (wave * 64 < BM) {
        const int64_t tok = m0 + wave * 64 + lane;
        const uint32_t off = (uint32_t)((tok < M ? tok : M - 1) * 16);
        dma16(ga.rec + (int64_t)hs * M * 16, off, lds_addr(&recL[hs % 4][wave * 64]));
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // v_mfma_f32_32x32x16_bf16: lane l holds A row l % 32 (B column l % 32),
  // K elements 8 (l / 32) .. +7 of the 16; D element q of lane l is row
  // 8 (q / 4) + 4 (l / 32) + q % 4, column l % 32. The W
  // fragment goes in as A and the E fragment as B, so D is the transposed
  // tile: lane l holds token row l % 32 and, per q / 4, the four consecutive
  // output columns 8 (q / 4) + 4 (l / 32) + 0..3 -- contiguous in memory.
  const int fr = lane & 31;
  // K steps per stage and their operand type: bf16 steps are 16 wide (one
  // 16-byte chunk per lane: logical chunk 2 s + lane / 32 of the row), FP8
  // steps 64 wide (two chunks per lane: 4 s + 2 (lane / 32) and the next);
  // a chunk sits at its logical index ^ swz(row).
  constexpr int KSTEP = F8 ? 64 : 16;
  constexpr int NS = BK / KSTEP;
  constexpr int CPF = F8 ? 2 : 1;               // 16-byte LDS reads per fragment
  using frag_t = typename std::conditional<F8, i32x8_t, bf16x8_t>::type;
  auto read_frag = [&](const uint8_t* rowp, int st) -> frag_t {
    if constexpr (F8) {
      const int c0 = 4 * st + 2 * (lane >> 5);
      const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((c0 ^ swz(fr)) * 16));
      const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((c0 + 1) ^ swz(fr)) * 16));
      return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      const int c = (st * 2 + (lane >> 5)) ^ swz(fr);
      return as_bf16x8(*reinterpret_cast<const uint4*>(rowp + c * 16));
    }
  };
  auto load_frags = [&](int kt, int st, frag_t (&af)[FM], frag_t (&bf)[FN]) {
    const uint8_t* sa = smem + (kt % S) * Cfg::kABytes;
    const uint8_t* sb = smem + Cfg::kBOffset + (kt % S) * Cfg::kBBytes;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = read_frag(sa + (wm * WTM + i * 32 + fr) * BKB, st);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = read_frag(sb + (wn * WTN + j * 32 + fr) * BKB, st);
  };
  auto mma = [&](const frag_t (&af)[FM], const frag_t (&bf)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (F8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bf[j], af[i], acc[i][j], 0, 0, 0, ep.f8_sa, 0, ep.f8_sb);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
      }
  };
  auto block_sync = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Rings of S buffers: stage kt+S-1 is loaded while stage kt is multiplied.
  // The barrier at the top of step kt means stage kt is in LDS and every wave
  // is done reading stage kt-1, whose buffers then take stage kt+S-1, issued
  // right there. Within a stage the fragment reads of K step st+1 go out one
  // after each MFMA of step st (LDS latency hides behind issued matrix work).
  // The epilogue's input tile (the residual x, or h) in registers: chunk q
  // of this thread is item tid + NT q of the row-major 8-column chunks. The
  // first PRE_EARLY chunks are requested at the top of the last K stage, so
  // their latency hides behind its matrix work (as many as the registers
  // allow beside the fragments); the rest before the epilogue's first pass.
  constexpr int R = Cfg::kPassRows;
  constexpr int NP = BM / R;                    // epilogue passes
  constexpr int ITEMS = R * CPR / NT;           // items per thread per pass
  static_assert(R * CPR % NT == 0, "epilogue items");
  constexpr int PRE_EARLY = BN <= 192 ? NP * ITEMS : ITEMS;
  // A full tile (every row and column inside, N a multiple of 8) takes the
  // branch-free path; edge tiles check each element.
  const bool full = m0 + BM <= M && n0 + BN <= N && (N & 7) == 0;
  uint4 pre[NP * ITEMS];
  auto load_pre = [&](int q0, int q1) {
#pragma unroll
    for (int q = 0; q < NP * ITEMS; ++q) {
      if (q < q0 || q >= q1) continue;
      if (pre_ok && full) {
        const int idx = tid + q * NT;
        pre[q] = *reinterpret_cast<const uint4*>(pre_src + (m0 + idx / CPR) * pre_ld + pre_c0 +
                                                 (idx % CPR) * 8);
      } else {
        pre[q] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  const int KT = K / BK;
  constexpr int PD = S - 1;                     // stages in flight
  constexpr int RD = (FM + FN) * CPF;           // LDS reads per step
  constexpr int NMF = FM * FN;                  // MFMAs per step
  constexpr int RPM = (RD + NMF - 1) / NMF;     // reads issued after each MFMA
  if constexpr (GATHER) {
    // the first records, and W's first stage (which waits for none)
    for (int hs = 0; hs < 3 && hs < KT; ++hs) issue_rec(hs);
    issue_b(0);
    wait_vmcnt<0>();
    __syncthreads();
    read_rows(0);
    issue_a(0);
    if (KT > 1) read_rows(1);
  } else {
#pragma unroll
    for (int st = 0; st < PD; ++st)
      if (st < KT) {
        issue_b(st);
        issue_a(st);
      }
  }
  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads of stage kt are done when at most the later issued
    // stages (up to PD - 1 of them) are outstanding
    const int later = KT - 1 - kt < PD - 1 ? KT - 1 - kt : PD - 1;
    if (later >= 2)
      wait_vmcnt<2 * L>();
    else if (later == 1)
      wait_vmcnt<L>();
    else
      wait_vmcnt<0>();
    block_sync();
    // the stage that reuses the buffers of stage kt-1 goes out at once, so
    // its load latency overlaps this stage's whole matrix work (fused
    // gather: after the records of head slot kt + 3, whose buffer was last
    // read in step kt - 1; the ring is then one stage deep, so the wait at
    // the top of the next step covers both; the rows of stage kt + 2 are
    // then read from their landed records)
    if (GATHER && kt + 3 < KT) issue_rec(kt + 3);
    if (kt + PD < KT) {
      issue_b(kt + PD);
      issue_a(kt + PD);
    }
    if (GATHER && kt + 2 < KT) read_rows(kt + 2);
    if (kt == KT - 1) load_pre(0, PRE_EARLY);
    // fused gather: this lane half's sign words of the stage's E rows
    uint32_t sgn[FM];
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        // the whole record in one 16-byte read: consecutive lanes read
        // consecutive records, free of bank conflicts (two 4-byte reads at
        // a 16-byte stride are not)
        uint4 r = recL[kt % 4][wm * WTM + i * 32 + fr];
        asm volatile("" : "+v"(r.x), "+v"(r.w));
        sgn[i] = lane < 32 ? r.y : r.z;
      }
    }
    // the bf16 sign bits (15 and 31) of dword q of K step st's fragment are
    // flipped by bits 15 - s and 31 - s of the sign word, s = 4 st + q
    auto apply_signs = [&](int st, frag_t (&af)[FM]) {
      if constexpr (GATHER) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          uint4 v = __builtin_bit_cast(uint4, af[i]);
          v.x ^= (sgn[i] << (4 * st)) & 0x80008000u;
          v.y ^= (sgn[i] << (4 * st + 1)) & 0x80008000u;
          v.z ^= (sgn[i] << (4 * st + 2)) & 0x80008000u;
          v.w ^= (sgn[i] << (4 * st + 3)) & 0x80008000u;
          af[i] = __builtin_bit_cast(frag_t, v);
        }
      }
    };
    frag_t fa[NS][FM], fb[NS][FN];
    load_frags(kt, 0, fa[0], fb[0]);
    apply_signs(0, fa[0]);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st + 1 < NS) {
        load_frags(kt, st + 1, fa[st + 1], fb[st + 1]);
        apply_signs(st + 1, fa[st + 1]);
      }
      mma(fa[st], fb[st]);
      if (st == 0) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
      if (st + 1 < NS) {
        // RPM reads after each MFMA until the step's RD reads are out
        constexpr int FULL = RD / RPM;          // MFMAs followed by RPM reads
        constexpr int REM = RD - FULL * RPM;    // reads after MFMA FULL
#pragma unroll
        for (int q = 0; q < FULL; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);   // RPM LDS reads
        }
        if constexpr (REM > 0) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, REM, 0);
        }
        constexpr int REST = NMF - FULL - (REM > 0 ? 1 : 0);
        if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      }
    }
  }

  // Epilogue: stage the accumulators through LDS, kPassRows rows at a time,
  // so global traffic is 16-byte loads and stores along rows. The passes
  // synchronise with LDS-only barriers: a __syncthreads() would also wait
  // for the previous pass's global stores. The scalar gate fetches its whole
  // residual tile before the first store (the fragment registers are free
  // by then), so no load is ever waited for behind a store.
  float* tile = reinterpret_cast<float*>(smem);
  constexpr int RS = Cfg::kRowStride;
  auto lds_barrier = [] {
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  load_pre(PRE_EARLY, NP * ITEMS);
  // Pass p: the accumulator rows [p R, p R + R) of the block tile go to LDS.
  auto stage = [&](int p) {
    lds_barrier();
    static_assert(R % 32 == 0, "a pass holds whole 32-row MFMA tiles");
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // wave-uniform: is this wave's 32-row tile i in pass p?
      if ((wm * WTM + i * 32) / R != p) continue;
      const int rl = wm * WTM + i * 32 + (lane & 31) - p * R;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = wn * WTN + j * 32 + 8 * g4 + 4 * (lane >> 5);
          *reinterpret_cast<float4*>(&tile[rl * RS + col]) =
              make_float4(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                          acc[i][j][4 * g4 + 3]);
        }
    }
    lds_barrier();
  };
  // Item it of pass p: tile row rl = (tid + 256 it) / CPR, columns c8..c8+7.
  auto item_y = [&](int p, int it, float (&y)[8], float (&xin)[8]) {
    const int idx = tid + it * NT;
    const int rl = idx / CPR;
    const int c8 = (idx - rl * CPR) * 8;
    const float4 lo = *reinterpret_cast<const float4*>(&tile[rl * RS + c8]);
    const float4 hi = *reinterpret_cast<const float4*>(&tile[rl * RS + c8 + 4]);
    y[0] = lo.x; y[1] = lo.y; y[2] = lo.z; y[3] = lo.w;
    y[4] = hi.x; y[5] = hi.y; y[6] = hi.z; y[7] = hi.w;
    const uint4 pr = pre[p * ITEMS + it];
    const uint32_t pw[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xin[2 * u] = bf16_to_f32((uint16_t)(pw[u] & 0xFFFFu));
      xin[2 * u + 1] = bf16_to_f32((uint16_t)(pw[u] >> 16));
    }
  };
  // The full-tile path is one straight line of passes (no join with the
  // edge path, whose loads would make every pass wait for earlier stores).
  if constexpr (EPI == EPI_F32) {
    float* obase0 = ep.out_f32 + (int64_t)blockIdx.y * M * ep.ldo;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      stage(p);
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int idx = tid + it * NT;
        const int64_t row = m0 + p * R + idx / CPR;
        const int col = n0 + (idx % CPR) * 8;
        float y[8], xin[8];
        item_y(p, it, y, xin);
        if (row >= M) continue;
        float* o = obase0 + row * ep.ldo + col;
        if (col + 8 <= N && (ep.ldo & 3) == 0) {
          *reinterpret_cast<float4*>(o) =
              make_float4(ep.g * y[0], ep.g * y[1], ep.g * y[2], ep.g * y[3]);
          *reinterpret_cast<float4*>(o + 4) =
              make_float4(ep.g * y[4], ep.g * y[5], ep.g * y[6], ep.g * y[7]);
        } else {
          for (int u = 0; u < 8 && col + u < N; ++u) o[u] = ep.g * y[u];
        }
      }
    }
  } else if constexpr (EPI == EPI_SCALAR) {
    if (full) {
      // Addresses: a wave-uniform row base per pass plus a 32-bit element
      // offset per item (the pass is R rows of N elements).
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        stage(p);
        uint16_t* obase = ep.out + (m0 + p * R) * (int64_t)N + n0;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
          const int idx = tid + it * NT;
          const uint32_t off = (uint32_t)((idx / CPR) * N + (idx % CPR) * 8);
          float y[8], xin[8];
          item_y(p, it, y, xin);
          uint32_t ow[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            ow[u] = pack_bf16x2(xin[2 * u] + ep.g * y[2 * u], xin[2 * u + 1] + ep.g * y[2 * u + 1]);
          *reinterpret_cast<uint4*>(obase + off) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        stage(p);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
          const int idx = tid + it * NT;
          const int64_t row = m0 + p * R + idx / CPR;
          const int col = n0 + (idx % CPR) * 8;
          float y[8], xin[8];
          item_y(p, it, y, xin);
          if (row >= M) continue;
          for (int u = 0; u < 8 && col + u < N; ++u) {
            const int64_t o = row * N + col + u;
            const float x = ep.resid ? bf16_to_f32(ep.resid[o]) : 0.f;
            ep.out[o] = (uint16_t)pack_bf16x2(x + ep.g * y[u], 0.f);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int S, int EPI, int MINB, int WGM, int WGN, bool F8>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_pipe_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Bw, int64_t M, int N,
    int K, EpiArgs ep) {
  const GatherArgs none{};
  pipe_body<BM, BN, BK, S, EPI, WGM, WGN, F8, false>(A, Bw, M, N, K, ep, none);
}

// pg_forward's fused path: the E operand gathered from the table.
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_pipe_gather_kernel(
    const uint8_t* __restrict__ Bw, int64_t M, int N, int K, EpiArgs ep, GatherArgs ga) {
  pipe_body<BM, BN, 64, 2, EPI_SCALAR, WGM, WGN, false, true>(nullptr, Bw, M, N, K, ep, ga);
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

// BM x BN tiles, K stages of BK elements through a ring of S, MINB blocks
// per CU, WGM x WGN waves per block; F8: E4M3 operands.
template <int BM, int BN, int BK, int S, int MINB, int EPI, int WGM = 2, int WGN = 2,
          bool F8 = false>
hipError_t launch_pipe(const void* e, int64_t M, int N, int K, const void* W,
                       const EpiArgs& ep, hipStream_t s, int splits = 1) {
  static_assert(PipeCfg<BM, BN, BK * (F8 ? 1 : 2), S>::kLdsBytes * MINB <= 160 * 1024,
                "LDS per CU");
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_pipe_kernel<BM, BN, BK, S, EPI, MINB, WGM, WGN, F8>),
                     dim3((unsigned)blocks, (unsigned)splits), dim3(64 * WGM * WGN), 0, s,
                     static_cast<const uint8_t*>(e), static_cast<const uint8_t*>(W), M, N, K,
                     ep);
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
  if (E % kPipeBK == 0) {
    // Pick the N tile by rounds of 256 concurrent blocks times block work.
    auto cost = [&](int64_t bn) {
      const int64_t blocks = ((N + 255) / 256) * ((d + bn - 1) / bn);
      return ((blocks + 255) / 256) * bn;
    };
    if (cost(192) < cost(256))
      return launch_pipe<256, 192, kPipeBK, kPipeStages, 1, EPI_SCALAR, 4, 2>(e, N, (int)d, (int)E, W, ep, s);
    return launch_pipe<256, 256, kPipeBK, kPipeStages, 1, EPI_SCALAR, 2, 4>(e, N, (int)d, (int)E, W, ep, s);
  }
  constexpr int BM = 128, BN = 128;
  const int64_t blocks = ((N + BM - 1) / BM) * ((d + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(e), static_cast<const uint16_t*>(W), N,
                     (int)d, (int)E, ep);
  return hipGetLastError();
}

// pg_forward's fused path (bf16 table with r = 64, scalar gate; checked by
// the caller): out[N][d] = resid + g * e W^T with e gathered in the kernel.
hipError_t launch_project_gathered(const void* table, const void* rec, int64_t N, int64_t E,
                                  const void* W, int64_t d, float g, const void* resid,
                                  void* out, hipStream_t s) {
  EpiArgs ep{};
  ep.g = g;
  ep.resid = static_cast<const uint16_t*>(resid);
  ep.out = static_cast<uint16_t*>(out);
  GatherArgs ga{};
  ga.table = static_cast<const uint8_t*>(table);
  ga.rec = static_cast<const uint8_t*>(rec);
  const auto* Wb = static_cast<const uint8_t*>(W);
  auto cost = [&](int64_t bn) {
    const int64_t blocks = ((N + 255) / 256) * ((d + bn - 1) / bn);
    return ((blocks + 255) / 256) * bn;
  };
  if (cost(192) < cost(256)) {
    const int64_t blocks = ((N + 255) / 256) * ((d + 191) / 192);
    hipLaunchKernelGGL((gemm_pipe_gather_kernel<256, 192, 4, 2>), dim3((unsigned)blocks),
                       dim3(512), 0, s, Wb, N, (int)d, E, ep, ga);
  } else {
    const int64_t blocks = ((N + 255) / 256) * ((d + 255) / 256);
    hipLaunchKernelGGL((gemm_pipe_gather_kernel<256, 256, 2, 4>), dim3((unsigned)blocks),
                       dim3(512), 0, s, Wb, N, (int)d, E, ep, ga);
  }
  return hipGetLastError();
}

// Scalar gate on FP8 operands: e8 [N][E] = E4M3(e 2^se), W8 [d][E] =
// E4M3(W 2^sw); E a multiple of 128 (checked by the caller).
hipError_t launch_project_scalar_fp8(const void* e8, int64_t N, int64_t E, const void* W8,
                                     int64_t d, float g, const void* resid, void* out,
                                     int se, int sw, hipStream_t s) {
  EpiArgs ep{};
  ep.g = g;
  ep.resid = static_cast<const uint16_t*>(resid);
  ep.out = static_cast<uint16_t*>(out);
  ep.f8_sa = 127 - sw;
  ep.f8_sb = 127 - se;
  auto cost = [&](int64_t bn) {
    const int64_t blocks = ((N + 255) / 256) * ((d + bn - 1) / bn);
    return ((blocks + 255) / 256) * bn;
  };
  if (cost(192) < cost(256))
    return launch_pipe<256, 192, kPipeBK8, kPipeStages, 1, EPI_SCALAR, 4, 2, true>(
        e8, N, (int)d, (int)E, W8, ep, s);
  return launch_pipe<256, 256, kPipeBK8, kPipeStages, 1, EPI_SCALAR, 2, 4, true>(
      e8, N, (int)d, (int)E, W8, ep, s);
}

// out[s][M][N] (fp32, row stride ldo) = g * A[M][s Kc .. (s+1) Kc) . B[N][same]^T
// for s < splits: bf16 operands with row strides lda / ldb; Kc a multiple of
// 64 (checked by the caller).
hipError_t launch_gemm_f32(const void* A, int lda, const void* B, int ldb, int64_t M, int N,
                           int Kc, int splits, float g, float* out, int64_t ldo,
                           hipStream_t s) {
  EpiArgs ep{};
  ep.g = g;
  ep.out_f32 = out;
  ep.ldo = ldo;
  ep.lda = lda;
  ep.ldb = ldb;
  return launch_pipe<256, 256, kPipeBK, kPipeStages, 1, EPI_F32, 2, 4>(A, M, N, Kc, B, ep, s, splits);
}

// Engram pass 1 (E % 64 == 0 and d % 256 == 0, checked by the caller; E %
// 128 == 0 for FP8 operands, f8 = 1 with scales se, sw): the slot-ring
// kernel of gemm_slots.hip for both operand types.
hipError_t launch_engram_pass1(const void* e, int64_t N, int64_t E, const void* W,
                               int64_t d, int64_t Mbr, const void* h,
                               const float* gamma_h, const float* gamma_k, uint16_t* v,
                               float* part_v, float* part_k, int f8, int se, int sw,
                               hipStream_t s) {
  return launch_engram_pass1_slots(e, N, E, W, d, Mbr, h, gamma_h, gamma_k, v, part_v, part_k,
                                   f8, se, sw, s);
}

}  // namespace pg
