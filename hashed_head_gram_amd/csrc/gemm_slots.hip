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
//
// With a slot count that is a multiple of 4 (bf16 or E4M3) the kernel is
// persistent: one block per CU walks its XCD's tiles, and each tile's
// epilogue turns the K walk to the next tile, whose gamma vectors and slots
// 0-2 load into the LDS the epilogue frees as it goes (slot k's buffer held
// h quarter k); slot 3 goes out at the next tile's start. So a tile's first
// slots are not a cold start. Wave 0 works out the next tile's coordinates
// at each tile's start and leaves them in LDS for the epilogue.
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

template <bool F8, bool P>
__global__ __launch_bounds__(512, 1) void engram_slot_kernel(const uint8_t* E,
                                                             const uint8_t* W,
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
  // P: the coordinates of the next tiles, two 32-byte records by tile parity
  constexpr int kNxtOff = kGamOff + 2 * BN * 4;
  constexpr int kLds = kNxtOff + (P ? 64 : 0);
  static_assert(E_DMA == 2 && W_DMA == 2, "two DMA instructions per operand and slot");
  static_assert(kLds <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];

  const int tid_k = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid_k >> 6), lane_k = tid_k & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  // Tiles are numbered so that each XCD (blocks are dealt round-robin to the
  // 8 XCDs) runs a contiguous range of them, walked in groups of 8 M tiles
  // N-major: concurrent tiles share their E and W panels in one L2. One
  // block per tile, or (P) one block per CU walking the tiles c, c + G/8,
  // c + 2 G/8, ... of its XCD's range (c = block / 8, G blocks; the few
  // tiles past 8 equal ranges go one each to the first blocks), so that the
  // next tile's first slots load while this one's epilogue runs.
  // (32-bit arithmetic: the tile counts fit, and 64-bit divisions by run-time
  // values expand to long scalar sequences every wave would run)
  const uint32_t nbm = (uint32_t)((M + BM - 1) / BM), nbn = (uint32_t)((N + BN - 1) / BN);
  const uint32_t total = nbm * nbn, per = total / 8;
  auto tile_id = [&](uint32_t j) -> uint32_t {
    if constexpr (P) {
      const uint32_t G8 = gridDim.x / 8, xcd = blockIdx.x & 7, cpos = blockIdx.x >> 3;
      const uint32_t n_main = cpos < per ? (per - cpos + G8 - 1) / G8 : 0;
      if (j < n_main) return xcd * per + cpos + G8 * j;
      if (j == n_main && blockIdx.x < total - 8 * per) return 8 * per + blockIdx.x;
      return 0xFFFFFFFFu;
    } else {
      uint32_t bid = blockIdx.x;
      if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
      return j == 0 ? bid : 0xFFFFFFFFu;
    }
  };
  uint32_t tile = tile_id(0);
  if (tile == 0xFFFFFFFFu) return;
  auto tile_bm_bn = [&](uint32_t id, uint32_t& bm, uint32_t& bn) {
    const uint32_t per_group = 8 * nbn, g = id / per_group, local = id - g * per_group;
    const uint32_t grows = nbm - g * 8 < 8 ? nbm - g * 8 : 8;
    bn = local / grows;
    bm = g * 8 + (local - bn * grows);
  };
  const int KS = K / SK;                   // slots (an even count: K a multiple of 2 SK)
  // the current tile (the epilogue's state) and its K walk (the DMA's state,
  // which the epilogue of a P block turns to the next tile)
  int64_t m0;
  int seg, cl0, s0;
  bool use_h, early_h;
  const uint16_t* hsrc;
  int64_t rbE, rbW;
  uint32_t offE[2], offW[2];
  auto phys = [&](int s) -> int64_t { return s + s0 < KS ? s + s0 : s + s0 - KS; };
  // Chunk c of a slot row r sits at c ^ swz(r): the 16 lanes a 16-byte read
  // serves together hit 16 distinct 16-byte slots of a 256-byte line.
  auto swz = [](int r) { return (r / ROWS_PER_LINE) & (LPR - 1); };
  const int dr = lane_k / LPR;
  const uint32_t chunk_b = (uint32_t)(((lane_k % LPR) ^ swz(dr)) * 16);
  uint32_t lds0 = lds_u32(smem);
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
  // The tiles that share an E panel (same bm) or a W panel (same bn) walk K
  // from different starting slots, one apart, so that of the tiles running
  // together only the first to ask for a panel's slot misses in L2 and the
  // others find it there a slot period later.
  // offE/offW hold the offsets of a tile inside M and N (the same for every
  // such tile): a walk between two of them keeps them
  bool offs_inner = false;
  auto set_walk = [&](uint32_t bm, uint32_t bn, int s0n) {
    s0 = s0n;
    const int64_t mE = (int64_t)bm * BM, mW = (int64_t)bn * BN;
    const bool inner = mE + BM <= M && mW + BN <= N;
    if (inner && offs_inner) {
      rbE = mE + wave * 2 * RPI;
      rbW = mW + wave * 2 * RPI;
    } else {
      rbE = dma_offsets(M, mE, offE);
      rbW = dma_offsets(N, mW, offW);
    }
    offs_inner = inner;
  };
  auto set_tile = [&](uint32_t bm, int sg, int c0) {
    m0 = (int64_t)bm * BM;
    seg = sg;                              // 0: v, m >= 1: k of branch m
    cl0 = c0;                              // first column within the segment
    use_h = seg > 0;
    hsrc = use_h ? ep.h + (int64_t)(seg - 1) * M * ep.d : ep.h;
    early_h = use_h && m0 + BM <= M;
  };
  {
    uint32_t bm, bn;
    tile_bm_bn(tile, bm, bn);
    const int n0 = (int)(bn * BN), sg = n0 / ep.d;
    set_tile(bm, sg, n0 - sg * ep.d);
    set_walk(bm, bn, (int)((bm + bn) % (uint32_t)KS));
  }
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
      const int p16 = lane_k & 31;
      const uint8_t* base =
          reinterpret_cast<const uint8_t*>(hsrc + (m0 + rw) * (int64_t)ep.d + cl0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rr = q * 2 + (lane_k >> 5);
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
  for (uint32_t jt = 0;; ++jt) {
    // P: values derived from these are recomputed per tile rather than held
    // across the epilogue (lane and tid shadow the kernel's own)
    int lane = lane_k, tid = tid_k;
    if constexpr (P) {
      asm volatile("" : "+s"(lds0));
      asm volatile("" : "+s"(E), "+s"(W));
      asm volatile("" : "+v"(lane), "+v"(tid));
    }
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
    auto issue_gamma = [&](bool uh, int c0) {
      if (uh && wave < 4) {
        dma4(ep.gamma_h + c0 + wave * 64, (uint32_t)lane * 4, lds0 + kGamOff + wave * 256);
        dma4(ep.gamma_k + c0 + wave * 64, (uint32_t)lane * 4, lds0 + kGamOff + BN * 4 + wave * 256);
      }
    };
    // a P block's later tiles had their gamma vectors and slots 0-2 requested
    // during the previous tile's epilogue (slot 3 goes out after the first
    // barrier below)
    const bool fresh = !P || jt == 0;
    if constexpr (P) {
      // wave 0 works out tile jt + 1 while the block waits for slot 0
      if (wave == 0) {
        const uint32_t id = tile_id(jt + 1);
        uint4 r0 = make_uint4(id, 0u, 0u, 0u), r1 = make_uint4(0u, 0u, 0u, 0u);
        if (id != 0xFFFFFFFFu) {
          uint32_t bm, bn;
          tile_bm_bn(id, bm, bn);
          const int n0 = (int)(bn * BN), sg = n0 / ep.d;
          r0 = make_uint4(id, bm, bn, (bm + bn) % (uint32_t)KS);
          r1 = make_uint4((uint32_t)sg, (uint32_t)(n0 - sg * ep.d), 0u, 0u);
        }
        if (lane == 0) {
          uint4* rec = reinterpret_cast<uint4*>(smem + kNxtOff + ((jt + 1) & 1) * 32);
          rec[0] = r0;
          rec[1] = r1;
        }
      }
    }
    if (fresh) issue_gamma(use_h, cl0);

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
      if (fresh) {
#pragma unroll
        for (int p = -4; p < 0; ++p) {
          issue_half(p, 0);
          issue_half(p, 1);
        }
        wait_slot(0, 0);
        bar();
      } else {
        // as in the bf16 loop below
        wait_vm<2 * LS>();
        bar();
        issue_half(-1, 0);
        issue_half(-1, 1);
      }
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
          af[i] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4*>(se + r * SKB + ((c ^ swz(r)) * 16)));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * WTN + j * 32 + fr;
          bf[j] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4*>(sw + r * SKB + ((c ^ swz(r)) * 16)));
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
      if (fresh) {
#pragma unroll
        for (int p = -4; p < 0; ++p) {
          issue_half(p, 0);
          issue_half(p, 1);
        }
        wait_slot(0, 0);
        bar();
      } else {
        // slots 0-2 came during the previous epilogue (anything issued after
        // them is older than what this wait needs); slot 3 goes out now, still
        // ahead of period 0, so the loop's counts hold
        wait_vm<2 * LS>();
        bar();
        issue_half(-1, 0);
        issue_half(-1, 1);
      }
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
          acc[0][0] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][0], fa[1][0], acc[0][0], 0, 0, 0);
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
    // P: the next tile's K walk replaces this one's (the loop is done with
    // it), from the record wave 0 wrote at this tile's start; its gamma
    // vectors and slots 0-2 go into the LDS this epilogue frees (slot k's
    // buffer holds h quarter k: KS is a multiple of 4), slot 3 at its start
    const uint4* nrec = reinterpret_cast<const uint4*>(smem + kNxtOff + ((jt + 1) & 1) * 32);
    bool has_next = false, uh_next = false;
    int cl0_next = 0;
    if constexpr (P) {
      const uint4 r0 = nrec[0], r1 = nrec[1];
      has_next = __builtin_amdgcn_readfirstlane(r0.x) != 0xFFFFFFFFu;
      if (has_next) {
        set_walk(__builtin_amdgcn_readfirstlane(r0.y), __builtin_amdgcn_readfirstlane(r0.z),
                 (int)__builtin_amdgcn_readfirstlane(r0.w));
        uh_next = (int)__builtin_amdgcn_readfirstlane(r1.x) > 0;
        cl0_next = (int)__builtin_amdgcn_readfirstlane(r1.y);
      }
    }
    // gamma vectors loaded by this wave for the next tile (counted by waits)
    const bool g_next = has_next && uh_next && wave < 4;
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
          // quarters) has landed from every wave; with a next tile, its gamma
          // vectors (after step 0) and slots 0 .. i - 2 (4 each) are later
          // as well: 8 loads, and 2 more where this wave loads gamma
          if (i == 0) {
            wait_vm<12>();
          } else if (has_next) {
            if (g_next)
              wait_vm<10>();
            else
              wait_vm<8>();
          } else {
            if (i == 1) wait_vm<8>();
            if (i == 2) wait_vm<4>();
            if (i == 3) wait_vm<0>();
          }
          bar();
          // the next tile's loads go out in two halves, around the first
          // column block's sums, so the waves do not stall on a full queue
          if (has_next) {
            if (i == 0)
              issue_gamma(uh_next, cl0_next);
            else
              issue_half(i - 1 - 4, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
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
          if (j == 1 && early_h && has_next && i > 0) {
            __builtin_amdgcn_sched_barrier(0);
            issue_half(i - 1 - 4, 1);
            __builtin_amdgcn_sched_barrier(0);
          }
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
    if (has_next) {
      // every wave is done with the ring and the gamma vectors
      // (slot 3 goes out at the next tile's start)
      if (!early_h) {
        issue_gamma(uh_next, cl0_next);
#pragma unroll
        for (int p = -4; p < -1; ++p) {
          issue_half(p, 0);
          issue_half(p, 1);
        }
      }
    }
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
    if (!has_next) break;
    {
      const uint4 r0 = nrec[0], r1 = nrec[1];
      set_tile(__builtin_amdgcn_readfirstlane(r0.y), (int)__builtin_amdgcn_readfirstlane(r1.x),
               (int)__builtin_amdgcn_readfirstlane(r1.y));
    }
  }
}

// Compute units of the current device, looked up once per device.
hipError_t cu_count(int* out) {
  constexpr int kMaxDev = 64;
  static int cached[kMaxDev];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < kMaxDev && cached[dev] > 0) {
    *out = cached[dev];
    return hipSuccess;
  }
  int n = 0;
  err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < kMaxDev) cached[dev] = n;
  *out = n;
  return hipSuccess;
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
  const int64_t KS = E / (f8 ? 64 : 32);
  const auto* ep8 = static_cast<const uint8_t*>(e);
  const auto* W8 = static_cast<const uint8_t*>(W);
  if (KS % 4 == 0) {
    // one block per CU (a multiple of 8 blocks, so every XCD has as many)
    int cus = 0;
    const hipError_t err = cu_count(&cus);
    if (err != hipSuccess) return err;
    int64_t grid = cus / 8 * 8;
    if (grid < 8) grid = 8;
    if (grid > (blocks + 7) / 8 * 8) grid = (blocks + 7) / 8 * 8;
    if (f8)
      hipLaunchKernelGGL((engram_slot_kernel<true, true>), dim3((unsigned)grid), dim3(512), 0, s,
                         ep8, W8, N, (int)Nout, (int)E, ep);
    else
      hipLaunchKernelGGL((engram_slot_kernel<false, true>), dim3((unsigned)grid), dim3(512), 0,
                         s, ep8, W8, N, (int)Nout, (int)E, ep);
  } else if (f8) {
    hipLaunchKernelGGL((engram_slot_kernel<true, false>), dim3((unsigned)blocks), dim3(512), 0,
                       s, ep8, W8, N, (int)Nout, (int)E, ep);
  } else {
    hipLaunchKernelGGL((engram_slot_kernel<false, false>), dim3((unsigned)blocks), dim3(512), 0,
                       s, ep8, W8, N, (int)Nout, (int)E, ep);
  }
  return hipGetLastError();
}

}  // namespace pg
