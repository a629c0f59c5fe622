// Projection GEMMs (gfx950).
//
// bf16: Y[M x N] = E[M x K] . W[N x K]^T on MFMA (v_mfma_f32_16x16x32_bf16,
// fp32 accumulation). Both operands are K-contiguous, the layout the MFMA A
// and B fragments want. 256 threads = 4 waves in a 2 x 2 grid; each wave
// owns a (BM/2) x (BN/2) sub-tile of 16 x 16 MFMA tiles. Tiles of BK = 64 go
// global -> registers -> LDS (rows padded by 16 bytes) with one tile in
// flight while the previous one is multiplied. Blocks are renumbered so that
// each XCD (blocks are dealt round-robin to the 8 XCDs) works on a
// contiguous range of M-major tiles, keeping an E tile and W in its L2.
//
// Epilogues: the scalar gate (PageGram §3.1: x + g W_V e), and pass 1 of
// the Engram fusion (Engram notes §3.3-3.4): v = W_V e is stored in bf16 and,
// per token and 128-column block, the partial sums that RMSNorm and the
// context gate need (sum v^2; per branch sum k^2, sum g_h g_k h k, sum h^2)
// are written to the workspace, so k is never stored.
//
// fp32: a plain LDS-tiled FMA GEMM for fp32 tables (tiny workloads).
#include "common.h"

namespace pg {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;   // padded LDS row (elements)

enum { EPI_SCALAR = 0, EPI_ENGRAM = 1 };

struct EpiArgs {
  // scalar gate
  float g;
  const uint16_t* resid;   // [M][N] or NULL
  uint16_t* out;           // [M][N]
  // Engram pass 1
  int d;
  int n_cb;                // d / BN column blocks per segment
  const uint16_t* h;       // [Mbr][M][d] or NULL
  uint16_t* v;             // [M][d]
  float* part_v;           // [n_cb][M]
  float* part_k;           // [Mbr][3][n_cb][M]
  const float* gamma_h;
  const float* gamma_k;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

template <int BM, int BN, int EPI>
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
  const int64_t total = nbm * nbn;
  int64_t bid = blockIdx.x;
  const int64_t per = total / 8;
  if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
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

  // Accumulator element (i, j, q) is row wm*WTM + i*16 + 4*(lane/16) + q,
  // column wn*WTN + j*16 + lane%16 of the block tile.
  if constexpr (EPI == EPI_SCALAR) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + q;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WTN + j * 16 + (lane & 15);
          if (col >= N) continue;
          const int64_t o = row * N + col;
          const float x = ep.resid ? bf16_to_f32(ep.resid[o]) : 0.f;
          ep.out[o] = f32_to_bf16(x + ep.g * acc[i][j][q]);
        }
      }
  } else {
    // Engram pass 1. BN divides d, so the tile lies in one segment:
    // s = 0 is v = W_V e, s = 1 + m is k^m = W_K^(m) e.
    __shared__ float red[2][BM][3];
    const int seg = n0 / ep.d;
    const int c0 = n0 - seg * ep.d;   // first column of the tile in its segment
    const int cb = c0 / BN;
    const int br = seg - 1;
    float s0[FM][4], s1[FM][4], s2[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s0[i][q] = 0.f;
        s1[i][q] = 0.f;
        s2[i][q] = 0.f;
        const int64_t row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + q;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = c0 + wn * WTN + j * 16 + (lane & 15);
          const float y = acc[i][j][q];
          if (seg == 0) {
            ep.v[row * ep.d + c] = f32_to_bf16(y);
            s0[i][q] += y * y;
          } else {
            const float hv = ep.h ? bf16_to_f32(ep.h[((int64_t)br * M + row) * ep.d + c]) : 0.f;
            s0[i][q] += y * y;
            s1[i][q] += ep.gamma_h[c] * ep.gamma_k[c] * hv * y;
            s2[i][q] += hv * hv;
          }
        }
      }
    // Reduce over the 16 lanes that share rows, then over the two wave columns.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int sh = 1; sh < 16; sh <<= 1) {
          s0[i][q] += __shfl_xor(s0[i][q], sh, 64);
          s1[i][q] += __shfl_xor(s1[i][q], sh, 64);
          s2[i][q] += __shfl_xor(s2[i][q], sh, 64);
        }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rl = wm * WTM + i * 16 + 4 * (lane >> 4) + q;
          red[wn][rl][0] = s0[i][q];
          red[wn][rl][1] = s1[i][q];
          red[wn][rl][2] = s2[i][q];
        }
    }
    __syncthreads();
    for (int rl = tid; rl < BM; rl += kThreads) {
      const int64_t row = m0 + rl;
      if (row >= M) continue;
      const float a0 = red[0][rl][0] + red[1][rl][0];
      if (seg == 0) {
        ep.part_v[(int64_t)cb * M + row] = a0;
      } else {
        const float a1 = red[0][rl][1] + red[1][rl][1];
        const float a2 = red[0][rl][2] + red[1][rl][2];
        float* pk = ep.part_k + (int64_t)br * 3 * ep.n_cb * M;
        pk[((int64_t)0 * ep.n_cb + cb) * M + row] = a0;
        pk[((int64_t)1 * ep.n_cb + cb) * M + row] = a1;
        pk[((int64_t)2 * ep.n_cb + cb) * M + row] = a2;
      }
    }
  }
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
  constexpr int BM = 128, BN = 128;
  EpiArgs ep{};
  ep.g = g;
  ep.resid = static_cast<const uint16_t*>(resid);
  ep.out = static_cast<uint16_t*>(out);
  const int64_t blocks = ((N + BM - 1) / BM) * ((d + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, EPI_SCALAR>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(e),
                     static_cast<const uint16_t*>(W), N, (int)d, (int)E, ep);
  return hipGetLastError();
}

// Engram pass 1 (declared in engram.hip's launcher).
hipError_t launch_engram_pass1(const void* e, int64_t N, int64_t E, const void* W,
                               int64_t d, int64_t Mbr, const void* h,
                               const float* gamma_h, const float* gamma_k, uint16_t* v,
                               float* part_v, float* part_k, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  EpiArgs ep{};
  ep.d = (int)d;
  ep.n_cb = (int)(d / BN);
  ep.h = static_cast<const uint16_t*>(h);
  ep.v = v;
  ep.part_v = part_v;
  ep.part_k = part_k;
  ep.gamma_h = gamma_h;
  ep.gamma_k = gamma_k;
  const int64_t Ntot = (1 + Mbr) * d;
  const int64_t blocks = ((N + BM - 1) / BM) * (Ntot / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, EPI_ENGRAM>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(e),
                     static_cast<const uint16_t*>(W), N, (int)Ntot, (int)E, ep);
  return hipGetLastError();
}

}  // namespace pg
