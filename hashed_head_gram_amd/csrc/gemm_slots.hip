// Pass 1 of the Engram fusion (gfx950): the fused projection
// [W_V; W_K^(1..M)] e with its partial-sum epilogue (Engram notes §3.3-3.4:
// v = W_V e is kept, k^m = W_K^m e only enters RMSNorm(k) and the context
// gate's dot product with RMSNorm(h), so per token and 256-column block the
// epilogue leaves sum v^2 and, per branch, sum k^2, sum gamma_h gamma_k h k
// and sum h^2; v goes out in bf16), on bf16 operands or on E4M3 ones with
// power-of-two scales (the FP8 GEMM the Engram notes §3.4 name).
//
// Y[M x N] = E[M x K] . W[N x K]^T, 256 x 256 block tiles, 512 threads = 8
// waves (two per SIMD) in a 2 x 4 grid of 128 x 64 wave tiles made of
// 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16, or
// v_mfma_scale_f32_32x32x64_f8f6f4 whose E8M0 operand scales undo the
// operands' scaling); the W fragment is the A operand, so a lane's
// accumulators are runs of four consecutive output columns of one token.
//
// K is walked in slots of 64 bytes per row (32 bf16 or 64 E4M3 elements)
// through a ring of four LDS slot buffers (16 KB of E rows and 16 KB of W
// rows each), filled by direct global->LDS loads (global_load_lds_dwordx4).
// The DMA of slot s + 4 goes into slot s's buffer as soon as every wave has
// read slot s, so three slots of loads stay in flight. bf16: two K steps per
// slot, fragments read one step ahead, the slot's DMA spread over its two
// steps and one block barrier per slot in its middle. E4M3: one K step per
// slot, the barrier at its start, the next slot's fragments read between
// the MFMAs into a second fragment set. Away from the first and last slots
// every DMA period loads a K slot, so those slots run a branch-free body:
// constant vmcnt waits, and the MFMAs after a barrier start before that
// period's DMA is issued. Each tile starts its walk over K at slot
// (bm + bn) mod KS, so the tiles sharing a panel ask for each slot a slot
// period apart instead of all at once (the sum order over K differs per tile).
//
// Epilogue without an accumulator round trip: as the last four slots' buffers
// free up, their DMA turns to the h tile of the block's branch (a quarter of
// the 256 x 256 bf16 tile each: quarter q holds the rows the waves handle in
// epilogue step q), so it is in LDS as the loop ends, and each step waits
// only for its own quarter. Each lane forms its partial sums straight from
// its accumulators and the h values of the same elements, one cross-lane add
// pairs the two half-waves holding a token's columns, and the four column
// waves meet in a small LDS table; gamma_h and gamma_k of the tile's columns
// come into LDS by DMA before the first slot. v tiles go out through LDS as
// 16-byte row stores (the ring is free by then). The h tile's and the v
// staging's 16-byte chunks sit at chunk ^ (row & 31) so a half-wave's reads
// of one column block hit distinct banks.
#include "common.h"

#include <type_traits>

namespace pg {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kColBlock = 256;

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Direct global->LDS load (see gemm.hip): 16 bytes per lane from base + off,
// the wave's 1 KiB to LDS address lds (M0). Not tracked by the compiler's
// wait counting; the ring orders it with explicit vmcnt waits and barriers.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds));
}
// The same with 4 bytes per lane (the wave's 256 bytes to LDS address lds).
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" : : "v"(off), "s"(base), "{m0}"(lds));
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

struct SlotEpi {
  int d;                   // columns per segment (d of the model)
  int n_cb;                // d / 256
  const uint16_t* h;       // [Mbr][M][d]
  uint16_t* v;             // [M][d]
  float* part_v;           // [n_cb][M]
  float* part_k;           // [Mbr][3][n_cb][M]
  const float* gamma_h;
  const float* gamma_k;
  int f8_sa, f8_sb;        // E8M0 operand scales of the E4M3 form (W, e)
};

template <bool F8>
__global__ __launch_bounds__(512, 1) void engram_slot_kernel(const uint8_t* __restrict__ E,
                                                             const uint8_t* __restrict__ W,
                                                             int64_t M, int N, int K,
                                                             SlotEpi ep) {
  // a slot is 64 bytes of every row: 32 bf16 or 64 E4M3 K elements
  constexpr int EB = F8 ? 1 : 2, SK = 64 / EB;
  constexpr int BM = 256, BN = 256, SKB = SK * EB, NSLOT = 4;
  constexpr int NT = 512, NW = 8, WGN = 4;
  constexpr int WTM = 128, WTN = 64, FM = WTM / 32, FN = WTN / 32;
  constexpr int LPR = SKB / 16, RPI = 64 / LPR, ROWS_PER_LINE = 256 / SKB;
  constexpr int E_DMA = BM / RPI / NW, W_DMA = BN / RPI / NW;   // per wave and slot
  constexpr int LS = E_DMA + W_DMA;
  constexpr int kSlotE = BM * SKB, kSlotW = BN * SKB;
  constexpr int kWOff = NSLOT * kSlotE;
  constexpr int kRingBytes = NSLOT * (kSlotE + kSlotW);
  constexpr int kRedOff = kRingBytes;
  constexpr int kGamOff = kRedOff + WGN * BM * 3 * 4;   // gamma_h, gamma_k of the 256 columns
  constexpr int kLds = kGamOff + 2 * BN * 4;
  static_assert(E_DMA == 2 && W_DMA == 2, "two DMA instructions per operand and slot");
  static_assert(kLds <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  // Blocks are renumbered so that each XCD (blocks are dealt round-robin to
  // the 8 XCDs) runs a contiguous range of tiles, walked in groups of 8 M
  // tiles N-major: concurrent tiles share their E and W panels in one L2.
  // (32-bit arithmetic: the tile counts fit, and 64-bit divisions by run-time
  // values expand to long scalar sequences every wave would run)
  const uint32_t nbm = (uint32_t)((M + BM - 1) / BM), nbn = (uint32_t)((N + BN - 1) / BN);
  uint32_t bid = blockIdx.x;
  {
    const uint32_t total = nbm * nbn, per = total / 8;
    if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
  }
  const uint32_t per_group = 8 * nbn, g = bid / per_group, local = bid - g * per_group;
  const uint32_t grows = nbm - g * 8 < 8 ? nbm - g * 8 : 8;
  const uint32_t bn = local / grows, bm = g * 8 + (local - bn * grows);
  const int64_t m0 = (int64_t)bm * BM;
  const int n0 = (int)(bn * BN);
  const int seg = n0 / ep.d;               // 0: v, m >= 1: k of branch m
  const int cl0 = n0 - seg * ep.d;         // first column within the segment
  const bool full = m0 + BM <= M;
  const bool use_h = seg > 0;
  const uint16_t* hsrc = use_h ? ep.h + (int64_t)(seg - 1) * M * ep.d : ep.h;
  const bool early_h = use_h && full;
  const int KS = K / SK;                   // slots (an even count: K a multiple of 2 SK)
  // The tiles that share an E panel (same bm) or a W panel (same bn) walk K
  // from different starting slots, one apart, so that of the tiles running
  // together only the first to ask for a panel's slot misses in L2 and the
  // others find it there a slot period later.
  const int s0 = (int)((bm + bn) % (uint32_t)KS);
  auto phys = [&](int s) -> int64_t { return s + s0 < KS ? s + s0 : s + s0 - KS; };

  // Chunk c of a slot row r sits at c ^ swz(r): the 16 lanes a 16-byte read
  // serves together hit 16 distinct 16-byte slots of a 256-byte line.
  auto swz = [](int r) { return (r / ROWS_PER_LINE) & (LPR - 1); };
  const int dr = lane / LPR;
  const uint32_t chunk_b = (uint32_t)(((lane % LPR) ^ swz(dr)) * 16);
  const uint32_t lds0 = lds_u32(smem);
  // instruction q of this wave loads rows r_base + q RPI + dr of an operand
  // (rows past its end repeat its last row, never stored); one SGPR base per
  // operand and slot, the row offsets are loop-invariant
  auto dma_offsets = [&](int64_t rows, int64_t r00, uint32_t (&off)[2]) -> int64_t {
    const int64_t r_base = r00 + (int64_t)wave * 2 * RPI;
    const int64_t rb = r_base < rows ? r_base : rows - 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t r = r_base + q * RPI + dr;
      const int64_t rc = r < rows ? r : rows - 1;
      off[q] = (uint32_t)((rc - rb) * K * EB) + chunk_b;
    }
    return rb;
  };
  uint32_t offE[2], offW[2];
  const int64_t rbE = dma_offsets(M, m0, offE);
  const int64_t rbW = dma_offsets(N, n0, offW);
  // h tile row r (0..255), 512 bytes a row: quarter q = (r / 32) & 3 holds
  // the rows that the waves' epilogue step q reads (rows 32 q .. +31 in the E
  // part of the buffer of slot KS - 4 + q, rows 128 + 32 q .. +31 in its W
  // part), so the epilogue can start on the quarters that landed first.
  auto hrow_off = [&](int r) -> uint32_t {
    const int b = (KS - 4 + ((r >> 5) & 3)) & 3;
    const int rr = r & 31;
    return (uint32_t)(r < 128 ? b * kSlotE + rr * 512 : kWOff + b * kSlotW + rr * 512);
  };
  // DMA period p (issued between the barriers of slots p and p + 1; the
  // prologue is periods -4 .. -1) loads slot p + 4 into slot p's buffer, or,
  // once the slots are out, quarter q = p + 4 - KS of the h tile; half 0 is
  // the E part (h rows 32 q .. +31), half 1 the W part (rows 128 + 32 q ..).
  auto period_count = [&](int p) -> int {
    const int s = p + 4;
    return (s < KS || (early_h && s - KS < 4)) ? LS : 0;
  };
  auto issue_half = [&](int p, int half) {
    const int s = p + 4;
    if (s < KS) {
      const int b = s & 3;
      if (half == 0) {
        const uint8_t* base = E + (rbE * K + phys(s) * SK) * EB;
        const uint32_t l = lds0 + b * kSlotE + wave * E_DMA * 1024;
        dma16(base, offE[0], l);
        dma16(base, offE[1], l + 1024);
      } else {
        const uint8_t* base = W + (rbW * K + phys(s) * SK) * EB;
        const uint32_t l = lds0 + kWOff + b * kSlotW + wave * W_DMA * 1024;
        dma16(base, offW[0], l);
        dma16(base, offW[1], l + 1024);
      }
    } else if (early_h && s - KS < 4) {
      // 32 rows: 4 per wave, 2 per instruction (lanes 0-31 and 32-63)
      const int rw = half * 128 + (s - KS) * 32 + wave * 4;
      const int p16 = lane & 31;
      const uint8_t* base = reinterpret_cast<const uint8_t*>(hsrc + (m0 + rw) * (int64_t)ep.d + cl0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rr = q * 2 + (lane >> 5);
        dma16(base, (uint32_t)(rr * ep.d * 2 + ((p16 ^ ((rw + rr) & 31)) * 16)),
              lds0 + hrow_off(rw + q * 2));
      }
    }
  };
  // issue_half for a period that loads a K slot (s + 4 < KS): no branch
  auto issue_slot_half = [&](int p, int half) {
    const int s = p + 4, b = s & 3;
    if (half == 0) {
      const uint8_t* base = E + (rbE * K + phys(s) * SK) * EB;
      const uint32_t l = lds0 + b * kSlotE + wave * E_DMA * 1024;
      dma16(base, offE[0], l);
      dma16(base, offE[1], l + 1024);
    } else {
      const uint8_t* base = W + (rbW * K + phys(s) * SK) * EB;
      const uint32_t l = lds0 + kWOff + b * kSlotW + wave * W_DMA * 1024;
      dma16(base, offW[0], l);
      dma16(base, offW[1], l + 1024);
    }
  };
  // this wave's loads of slot s have landed when only those of the periods
  // after the one that issued it (s - 4), up to p_now - 1, are outstanding
  auto wait_slot = [&](int s, int p_now) {
    int later = 0;
    for (int p = s - 3; p < p_now; ++p) later += period_count(p);
    if (later >= 3 * LS)
      wait_vm<3 * LS>();
    else if (later >= 2 * LS)
      wait_vm<2 * LS>();
    else if (later >= LS)
      wait_vm<LS>();
    else
      wait_vm<0>();
  };
  auto bar = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lgkm0 = [] { __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14)); };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // k tiles: gamma_h and gamma_k of the tile's 256 columns go to LDS by DMA
  // ahead of the first slot (waves 0-3, 64 columns each), so the epilogue
  // issues no global load and can wait on its h quarters one by one; the
  // prologue's wait for slot 0 covers them
  if (use_h && wave < 4) {
    dma4(ep.gamma_h + cl0 + wave * 64, (uint32_t)lane * 4, lds0 + kGamOff + wave * 256);
    dma4(ep.gamma_k + cl0 + wave * 64, (uint32_t)lane * 4, lds0 + kGamOff + BN * 4 + wave * 256);
  }

  if constexpr (F8) {
    // v_mfma_scale_f32_32x32x64_f8f6f4: lane l holds operand row l % 32 and K
    // elements 32 (l / 32) .. +31 of the slot (two 16-byte chunks); D as for
    // the bf16 form. One MFMA K step per slot: barrier B_s at the slot's start
    // (slot s + 1 landed everywhere, every read of slot s done), period s's
    // loads into slot s's buffer, then slot s's MFMAs with slot s + 1's
    // fragment reads between them, into the other of two fragment sets (the
    // loop runs two slots per iteration, so the set is a constant). The last
    // slot also reads the next buffer; those values are never used.
    const int fr = lane & 31;
    i32x8_t fa[2][FM], fb[2][FN];
    auto read8 = [&](const uint8_t* rowp, int r) -> i32x8_t {
      const int c0 = 2 * (lane >> 5);
      const uint4 lo = *reinterpret_cast<const uint4*>(rowp + ((c0 ^ swz(r)) * 16));
      const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((c0 + 1) ^ swz(r)) * 16));
      return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto read_slot = [&](int s, i32x8_t (&af)[FM], i32x8_t (&bf)[FN]) {
      const uint8_t* se = smem + (s & 3) * kSlotE;
      const uint8_t* sw = smem + kWOff + (s & 3) * kSlotW;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + fr;
        af[i] = read8(se + r * SKB, r);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 32 + fr;
        bf[j] = read8(sw + r * SKB, r);
      }
    };
    auto f8_mma = [&](int i, int j, const i32x8_t (&af)[FM], const i32x8_t (&bf)[FN]) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af[i], acc[i][j], 0, 0,
                                                                   0, ep.f8_sa, 0, ep.f8_sb);
    };
    // kSteady: slot s + 1 exists and periods s - 2 .. s all load K slots, so
    // the wait is a constant and the slot's MFMAs start right after the
    // barrier, its DMA going out behind the first one
    auto f8_slot = [&](int s, i32x8_t (&af)[FM], i32x8_t (&bf)[FN], i32x8_t (&an)[FM],
                       i32x8_t (&bnx)[FN], auto steady) {
      constexpr bool kSteady = decltype(steady)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kSteady)
        wait_vm<2 * LS>();
      else if (s + 1 < KS)
        wait_slot(s + 1, s);
      lgkm0();
      bar();
      if constexpr (kSteady) {
        f8_mma(0, 0, af, bf);
        __builtin_amdgcn_sched_barrier(0);
        issue_slot_half(s, 0);
        issue_slot_half(s, 1);
        __builtin_amdgcn_sched_barrier(0);
        read_slot(s + 1, an, bnx);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (i + j > 0) f8_mma(i, j, af, bf);
        // two 16-byte reads before each of the next six MFMAs
#pragma unroll
        for (int x = 0; x < FM + FN; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - 1 - (FM + FN), 0);
      } else {
        issue_half(s, 0);
        issue_half(s, 1);
        __builtin_amdgcn_sched_barrier(0);
        read_slot(s + 1, an, bnx);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) f8_mma(i, j, af, bf);
        // two 16-byte reads after each of the first six MFMAs
#pragma unroll
        for (int x = 0; x < FM + FN; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: periods -4 .. -1 (slots 0-3); slot 0 landed; its fragments read
#pragma unroll
    for (int p = -4; p < 0; ++p) {
      issue_half(p, 0);
      issue_half(p, 1);
    }
    wait_slot(0, 0);
    bar();
    read_slot(0, fa[0], fb[0]);
    using steady_t = std::integral_constant<bool, true>;
    using generic_t = std::integral_constant<bool, false>;
    int s = 0;
    for (; s + 5 < KS; s += 2) {
      f8_slot(s, fa[0], fb[0], fa[1], fb[1], steady_t{});
      f8_slot(s + 1, fa[1], fb[1], fa[0], fb[0], steady_t{});
    }
    for (; s < KS; s += 2) {
      f8_slot(s, fa[0], fb[0], fa[1], fb[1], generic_t{});
      f8_slot(s + 1, fa[1], fb[1], fa[0], fb[0], generic_t{});
    }
  } else {

    // v_mfma_f32_32x32x16_bf16: lane l holds operand row l % 32 and K elements
    // 8 (l / 32) .. +7 of the step; D element q of lane l is row 8 (q / 4) +
    // 4 (l / 32) + q % 4 (an output column), column l % 32 (a token).
    const int fr = lane & 31;
    bf16x8_t fa[2][FM], fb[2][FN];
    auto load_step = [&](int s, int t, bf16x8_t (&af)[FM], bf16x8_t (&bf)[FN]) {
      const int b = s & 3;
      const uint8_t* se = smem + b * kSlotE;
      const uint8_t* sw = smem + kWOff + b * kSlotW;
      const int c = t * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + fr;
        af[i] = __builtin_bit_cast(bf16x8_t,
                                   *reinterpret_cast<const uint4*>(se + r * SKB + ((c ^ swz(r)) * 16)));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 32 + fr;
        bf[j] = __builtin_bit_cast(bf16x8_t,
                                   *reinterpret_cast<const uint4*>(sw + r * SKB + ((c ^ swz(r)) * 16)));
      }
    };
    auto mma_step = [&](const bf16x8_t (&af)[FM], const bf16x8_t (&bf)[FN], bool reads) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
      // the step's fragment reads go out one after each of its first MFMAs
      if (reads) {
#pragma unroll
        for (int x = 0; x < FM + FN; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      }
    };

    // prologue: periods -4 .. -1 (slots 0-3); slot 0 landed; its step 0 read
#pragma unroll
    for (int p = -4; p < 0; ++p) {
      issue_half(p, 0);
      issue_half(p, 1);
    }
    wait_slot(0, 0);
    bar();
    load_step(0, 0, fa[0], fb[0]);

    // Step (s, 0): reads of (s, 1), MFMAs of (s, 0), the second half of period
    // s - 1. Barrier B_s: slot s + 1 has landed everywhere and slot s is read.
    // Step (s, 1): the first half of period s, reads of (s + 1, 0), MFMAs.
    // kSteady (0 < s < KS - 4): both DMA periods of the slot load K slots
    // and slot s + 1 exists, so the wait is a constant, nothing branches, and
    // step (s, 1) starts its MFMAs right after the barrier with the period's
    // DMA behind the first one.
    auto slot = [&](int s, auto steady) {
      constexpr bool kSteady = decltype(steady)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kSteady)
        issue_slot_half(s - 1, 1);
      else if (s > 0)
        issue_half(s - 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      load_step(s, 1, fa[1], fb[1]);
      mma_step(fa[0], fb[0], true);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kSteady)
        wait_vm<2 * LS>();
      else if (s + 1 < KS)
        wait_slot(s + 1, s);
      lgkm0();
      bar();
      if constexpr (kSteady) {
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][0], fa[1][0], acc[0][0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue_slot_half(s, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_step(s + 1, 0, fa[0], fb[0]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (i + j > 0)
              acc[i][j] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][j], fa[1][i], acc[i][j], 0, 0, 0);
        // one read before each of the next six MFMAs
#pragma unroll
        for (int x = 0; x < FM + FN; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - 1 - (FM + FN), 0);
      } else {
        issue_half(s, 0);
        __builtin_amdgcn_sched_barrier(0);
        const bool rd = s + 1 < KS;
        if (rd) load_step(s + 1, 0, fa[0], fb[0]);
        mma_step(fa[1], fb[1], rd);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using steady_t = std::integral_constant<bool, true>;
    using generic_t = std::integral_constant<bool, false>;
    slot(0, generic_t{});
    int s = 1;
    for (; s < KS - 4; ++s) slot(s, steady_t{});
    for (; s < KS; ++s) slot(s, generic_t{});
    issue_half(KS - 1, 1);
  }

  // ---- epilogue
  auto lds_barrier = [] {
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int hl = lane >> 5;   // which 4-column half of each 8-column group
  float* red = reinterpret_cast<float*>(smem + kRedOff);   // [wn][256 rows][3]
  if (use_h) {
    // this lane's columns within the segment: cl0 + wn 64 + j 32 + 8 g4 + 4 hl + u
    const float* gH = reinterpret_cast<const float*>(smem + kGamOff);
    const float* gK = gH + BN;
    float gg[FN][4][4];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = wn * WTN + j * 32 + 8 * g4 + 4 * hl;
        const float4 a = *reinterpret_cast<const float4*>(gH + c);
        const float4 b = *reinterpret_cast<const float4*>(gK + c);
        gg[j][g4][0] = a.x * b.x;
        gg[j][g4][1] = a.y * b.y;
        gg[j][g4][2] = a.z * b.z;
        gg[j][g4][3] = a.w * b.w;
      }
    if (!early_h) {
      wait_vm<0>();
      bar();   // every slot has been read
      // edge tile: h rows straight into the freed ring (zeros past M)
      for (int idx = tid; idx < BM * 32; idx += NT) {
        const int r = idx >> 5, c = idx & 31;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (m0 + r < M)
          val = *reinterpret_cast<const uint4*>(hsrc + (m0 + r) * (int64_t)ep.d + cl0 + c * 8);
        *reinterpret_cast<uint4*>(smem + hrow_off(r) + ((c ^ (r & 31)) * 16)) = val;
      }
      lds_barrier();
    }
    static_assert(FM == 4, "one h quarter per row block");
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (early_h) {
        // quarter i (this wave's last 4 (3 - i) DMA instructions are later
        // quarters) has landed from every wave
        if (i == 0) wait_vm<12>();
        if (i == 1) wait_vm<8>();
        if (i == 2) wait_vm<4>();
        if (i == 3) wait_vm<0>();
        bar();
      }
      const int rl = wm * WTM + i * 32 + (lane & 31);
      const uint8_t* hrow = smem + hrow_off(rl) + hl * 8;
      // this row block's accumulators, copied out of the accumulator registers
      // here and nowhere else
      f32x16_t av[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        av[j] = acc[i][j];
        asm volatile("" : "+v"(av[j]));
      }
      float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        uint2 hv[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int chunk = wn * 8 + j * 4 + g4;
          hv[g4] = *reinterpret_cast<const uint2*>(hrow + ((chunk ^ (rl & 31)) * 16));
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float h4[4] = {__uint_as_float(hv[g4].x << 16),
                               __uint_as_float(hv[g4].x & 0xFFFF0000u),
                               __uint_as_float(hv[g4].y << 16),
                               __uint_as_float(hv[g4].y & 0xFFFF0000u)};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float y = av[j][4 * g4 + u];
            s0 += y * y;
            s1 += gg[j][g4][u] * h4[u] * y;
            s2 += h4[u] * h4[u];
          }
        }
      }
      s0 += __shfl_xor(s0, 32, 64);
      s1 += __shfl_xor(s1, 32, 64);
      s2 += __shfl_xor(s2, 32, 64);
      if (lane < 32) {
        float* rp = red + (wn * BM + rl) * 3;
        rp[0] = s0;
        rp[1] = s1;
        rp[2] = s2;
      }
    }
  } else {
    // v tile: bf16 v through the freed ring (rows of 512 bytes, chunk c at
    // c ^ (row & 31)), then 16-byte row stores
    wait_vm<0>();
    bar();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rl = wm * WTM + i * 32 + (lane & 31);
      f32x16_t av[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        av[j] = acc[i][j];
        asm volatile("" : "+v"(av[j]));
      }
      float s0 = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float y0 = av[j][4 * g4], y1 = av[j][4 * g4 + 1];
          const float y2 = av[j][4 * g4 + 2], y3 = av[j][4 * g4 + 3];
          s0 += y0 * y0 + y1 * y1 + y2 * y2 + y3 * y3;
          const int chunk = wn * 8 + j * 4 + g4;
          *reinterpret_cast<uint2*>(smem + rl * 512 + ((chunk ^ (rl & 31)) * 16) + hl * 8) =
              make_uint2(pack2(y0, y1), pack2(y2, y3));
        }
      s0 += __shfl_xor(s0, 32, 64);
      if (lane < 32) red[(wn * BM + rl) * 3] = s0;
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < BM * 32 / NT; ++q) {
      const int idx = tid + q * NT;
      const int r = idx >> 5, c = idx & 31;
      const uint4 val = *reinterpret_cast<const uint4*>(smem + r * 512 + ((c ^ (r & 31)) * 16));
      if (m0 + r < M)
        *reinterpret_cast<uint4*>(ep.v + (m0 + r) * (int64_t)ep.d + cl0 + c * 8) = val;
    }
  }
  lds_barrier();
  if (tid < BM) {
    const int64_t row = m0 + tid;
    if (row < M) {
      float t0 = 0.f, t1 = 0.f, t2 = 0.f;
#pragma unroll
      for (int w = 0; w < WGN; ++w) {
        const float* rp = red + (w * BM + tid) * 3;
        t0 += rp[0];
        t1 += rp[1];
        t2 += rp[2];
      }
      const int cb = cl0 / kColBlock;
      if (!use_h) {
        ep.part_v[(int64_t)cb * M + row] = t0;
      } else {
        float* pk = ep.part_k + (int64_t)(seg - 1) * 3 * ep.n_cb * M;
        pk[((int64_t)0 * ep.n_cb + cb) * M + row] = t0;
        pk[((int64_t)1 * ep.n_cb + cb) * M + row] = t1;
        pk[((int64_t)2 * ep.n_cb + cb) * M + row] = t2;
      }
    }
  }
}

}  // namespace

// Pass 1: e [N][E], W [(1 + Mbr) d][E], bf16 (E a multiple of 64) or, with
// f8, E4M3 with power-of-two scales 2^se (e) and 2^sw (W) (E a multiple of
// 128); d a multiple of 256 (checked by the caller).
hipError_t launch_engram_pass1_slots(const void* e, int64_t N, int64_t E, const void* W,
                                     int64_t d, int64_t Mbr, const void* h,
                                     const float* gamma_h, const float* gamma_k, uint16_t* v,
                                     float* part_v, float* part_k, int f8, int se, int sw,
                                     hipStream_t s) {
  SlotEpi ep{};
  ep.d = (int)d;
  ep.n_cb = (int)(d / kColBlock);
  ep.h = static_cast<const uint16_t*>(h);
  ep.v = v;
  ep.part_v = part_v;
  ep.part_k = part_k;
  ep.gamma_h = gamma_h;
  ep.gamma_k = gamma_k;
  ep.f8_sa = 127 - sw;
  ep.f8_sb = 127 - se;
  const int64_t Nout = (1 + Mbr) * d;
  const int64_t blocks = ((N + 255) / 256) * ((Nout + 255) / 256);
  if (f8)
    hipLaunchKernelGGL(engram_slot_kernel<true>, dim3((unsigned)blocks), dim3(512), 0, s,
                       static_cast<const uint8_t*>(e), static_cast<const uint8_t*>(W), N,
                       (int)Nout, (int)E, ep);
  else
    hipLaunchKernelGGL(engram_slot_kernel<false>, dim3((unsigned)blocks), dim3(512), 0, s,
                       static_cast<const uint8_t*>(e), static_cast<const uint8_t*>(W), N,
                       (int)Nout, (int)E, ep);
  return hipGetLastError();
}

}  // namespace pg
