// Engram fusion after the projection GEMM's pass 1 (gfx950): a per-token gate
// kernel, then pass 2.
//
// Engram notes §3.3-3.4 with M branches sharing v = W_V e:
//   alpha^m_t = sigmoid(RMSNorm_h(h^m_t) . RMSNorm_k(k^m_t) / sqrt(d))
//   u^m_t     = alpha^m_t v_t
//   z^m_t     = RMSNorm_u(u^m_t) = gamma_u * v_t * alpha / sqrt(alpha^2 ms(v_t) + eps)
//   out^m_t   = h^m_t + u^m_t + SiLU(sum_j w_j * z^m_{t-(kw-1-j)*dil})
// From pass 1 the workspace holds v (bf16) and per-token partial sums over
// 256-column blocks: sum v^2, and per branch sum k^2, sum gamma_h gamma_k h k,
// sum h^2. RMSNorm_h(h).RMSNorm_k(k) = that dot / (rms(h) rms(k)).
//
// The gate kernel reduces those partials once per (branch, token) into alpha
// and the RMSNorm_u scale alpha / sqrt(alpha^2 mean(v^2) + eps). Pass 2 takes
// TB tokens of one sequence and 256 channels per block, stages the v window
// (its tokens and the (kw-1)*dil before them) and their gate values in LDS,
// and each lane produces 8 channels of one token for all branches with
// 16-byte loads of h and stores of out.
#include "common.h"

namespace pg {

namespace {

constexpr int kThreads = 256;
constexpr int kTB = 32;          // tokens per block
constexpr int kCB = 256;         // channels per block
constexpr int kMaxBranches = 8;  // largest M (validated by the caller)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kTPT = kTB / (kThreads / 32);   // tokens per thread in pass 2

// Two floats to packed bf16 (round to nearest even, v_cvt_pk_bf16_f32); a low.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Eight bf16 (16 bytes, element 0 in the low half of the first word) to fp32.
__device__ __forceinline__ void unpack8(uint4 raw, float (&v)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    v[2 * x] = __uint_as_float(w[x] << 16);
    v[2 * x + 1] = __uint_as_float(w[x] & 0xFFFF0000u);
  }
}
constexpr int kColBlock = 256;   // pass-1 column block of the partial sums

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// gate[m][0][tok] = alpha, gate[m][1][tok] = alpha / sqrt(alpha^2 ms(v) + eps).
__global__ __launch_bounds__(kThreads) void engram_gate_kernel(
    int64_t N, int d, int Mbr, float eps, const float* __restrict__ part_v,
    const float* __restrict__ part_k, int n_cb, float* __restrict__ gate) {
  const int64_t tok = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int m = blockIdx.y;
  if (tok >= N) return;
  const float inv_d = 1.0f / (float)d;
  float sv = 0.f, sk = 0.f, dot = 0.f, sh = 0.f;
  const float* pk = part_k + (int64_t)m * 3 * n_cb * N;
  for (int cb = 0; cb < n_cb; ++cb) {
    sv += part_v[(int64_t)cb * N + tok];
    sk += pk[((int64_t)0 * n_cb + cb) * N + tok];
    dot += pk[((int64_t)1 * n_cb + cb) * N + tok];
    sh += pk[((int64_t)2 * n_cb + cb) * N + tok];
  }
  const float rk = 1.0f / sqrtf(sk * inv_d + eps);
  const float rh = 1.0f / sqrtf(sh * inv_d + eps);
  const float zlogit = dot * rh * rk / sqrtf((float)d);
  const float alpha = 1.0f / (1.0f + expf(-zlogit));
  gate[((int64_t)m * 2 + 0) * N + tok] = alpha;
  gate[((int64_t)m * 2 + 1) * N + tok] = alpha / sqrtf(alpha * alpha * (sv * inv_d) + eps);
}

// Dynamic LDS: v window [(TB + H) x 256] bf16, then alpha and the RMSNorm_u
// scale [M][TB + H] fp32.
template <int KW, int MAXB>
__global__ __launch_bounds__(kThreads) void engram_pass2_kernel(
    int64_t T, int d, int Mbr, const float* __restrict__ gamma_u,
    const float* __restrict__ conv_w, int dil, const uint16_t* __restrict__ v,
    const float* __restrict__ gate, int64_t N, const uint16_t* __restrict__ h,
    uint16_t* __restrict__ out, int add_resid) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  constexpr int kw = KW;
  const int H = (kw - 1) * dil;
  const int rowsL = kTB + H;
  uint16_t* vt = reinterpret_cast<uint16_t*>(dsm);
  float* alphaS = reinterpret_cast<float*>(dsm + rowsL * kCB * 2);
  float* facS = alphaS + Mbr * rowsL;

  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kTB;
  const int c0 = blockIdx.z * kCB;
  const int tid = threadIdx.x;

  // Gate values for positions t0-H .. t0+TB-1 (LDS index tau - (t0-H)).
  for (int q = tid; q < rowsL * Mbr; q += kThreads) {
    const int m = q / rowsL;
    const int tl = q - m * rowsL;
    const int64_t tau = t0 - H + tl;
    float alpha = 0.f, fac = 0.f;
    if (tau >= 0 && tau < T) {
      const int64_t tok = b * T + tau;
      alpha = gate[((int64_t)m * 2 + 0) * N + tok];
      fac = gate[((int64_t)m * 2 + 1) * N + tok];
    }
    alphaS[m * rowsL + tl] = alpha;
    facS[m * rowsL + tl] = fac;
  }
  // v window [t0-H, t0+TB) x [c0, c0+256), zeros outside the sequence.
  for (int q = tid; q < rowsL * (kCB / 8); q += kThreads) {
    const int tl = q / (kCB / 8);
    const int ch = (q - tl * (kCB / 8)) * 8;
    const int64_t tau = t0 - H + tl;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (tau >= 0 && tau < T && c0 + ch < d)
      val = *reinterpret_cast<const uint4*>(v + (b * T + tau) * d + c0 + ch);
    *reinterpret_cast<uint4*>(&vt[tl * kCB + ch]) = val;
  }
  __syncthreads();

  const int cg = tid & 31;
  const int c = c0 + cg * 8;
  if (c >= d) return;
  // Every h row this thread needs (its kTPT tokens, all branches) is requested
  // before any arithmetic or store, so a wave keeps MAXB * kTPT 16-byte loads
  // in flight (stores share the load counter on this GPU, so a load issued
  // after a store would also wait for it). h and out are streamed once:
  // non-temporal loads and stores.
  u32x4 hr[MAXB][kTPT];
#pragma unroll
  for (int m = 0; m < MAXB; ++m)
#pragma unroll
    for (int k = 0; k < kTPT; ++k) {
      const int64_t t = t0 + (tid >> 5) + k * (kThreads / 32);
      if (m < Mbr && t < T && add_resid)
        hr[m][k] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(h + (((int64_t)m * N + b * T + t) * d + c)));
      else
        hr[m][k] = u32x4{0u, 0u, 0u, 0u};
    }
  // conv weights with the RMSNorm_u gain folded in: wg = w * gamma_u
  float wg[8][kw];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const float gu = gamma_u[c + x];
#pragma unroll
    for (int j = 0; j < kw; ++j) wg[x][j] = conv_w[(c + x) * kw + j] * gu;
  }
#pragma unroll
  for (int k = 0; k < kTPT; ++k) {
    const int tl = (tid >> 5) + k * (kThreads / 32);
    const int64_t t = t0 + tl;
    if (t >= T) break;
    const int li = tl + H;  // LDS index of t
    float vc[8];
    unpack8(*reinterpret_cast<const uint4*>(&vt[li * kCB + cg * 8]), vc);
    // the kw taps' v values (shared by the branches)
    float vj[kw][8];
#pragma unroll
    for (int j = 0; j < kw; ++j)
      unpack8(*reinterpret_cast<const uint4*>(&vt[(li - (kw - 1 - j) * dil) * kCB + cg * 8]),
              vj[j]);
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      if (m >= Mbr) break;
      float conv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kw; ++j) {
        const float f = facS[m * rowsL + li - (kw - 1 - j) * dil];   // 0 before the start
#pragma unroll
        for (int x = 0; x < 8; ++x) conv[x] += wg[x][j] * (vj[j][x] * f);
      }
      const float alpha = alphaS[m * rowsL + li];
      float hv[8];
      unpack8(make_uint4(hr[m][k][0], hr[m][k][1], hr[m][k][2], hr[m][k][3]), hv);
      u32x4 res;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // SiLU(y) = y / (1 + e^-y)
        const float y0 = conv[2 * x] * __builtin_amdgcn_rcpf(1.0f + __expf(-conv[2 * x]));
        const float y1 =
            conv[2 * x + 1] * __builtin_amdgcn_rcpf(1.0f + __expf(-conv[2 * x + 1]));
        res[x] = pack_bf16x2(hv[2 * x] + (alpha * vc[2 * x] + y0),
                             hv[2 * x + 1] + (alpha * vc[2 * x + 1] + y1));
      }
      const int64_t o = ((int64_t)m * N + b * T + t) * d + c;
      __builtin_nontemporal_store(res, reinterpret_cast<u32x4*>(out + o));
    }
  }
}

}  // namespace

int64_t engram_workspace_bytes(int64_t N, int64_t d, int64_t M) {
  const int64_t n_cb = d / kColBlock;
  return align256(N * d * 2) + align256(n_cb * N * 4) + align256(M * 3 * n_cb * N * 4) +
         align256(M * 2 * N * 4);
}

namespace {

// The workspace's regions: v [N][d] bf16, sum v^2 partials [n_cb][N], per
// branch (sum k^2, sum gamma_h gamma_k h k, sum h^2) partials
// [M][3][n_cb][N], gates [M][2][N] (alpha, RMSNorm_u scale).
struct EngramWs {
  uint16_t* v;
  float* part_v;
  float* part_k;
  float* gate;
};

EngramWs engram_ws(void* workspace, int64_t N, int64_t d, int64_t M) {
  const int64_t n_cb = d / kColBlock;
  auto* base = static_cast<uint8_t*>(workspace);
  EngramWs w;
  w.v = reinterpret_cast<uint16_t*>(base);
  base += align256(N * d * 2);
  w.part_v = reinterpret_cast<float*>(base);
  base += align256(n_cb * N * 4);
  w.part_k = reinterpret_cast<float*>(base);
  base += align256(M * 3 * n_cb * N * 4);
  w.gate = reinterpret_cast<float*>(base);
  return w;
}

}  // namespace

hipError_t launch_engram_project(const void* e, int64_t N, int64_t E, const void* W, int64_t d,
                                 int64_t M, const float* gamma_h, const float* gamma_k,
                                 const void* h, void* workspace, int f8, int se, int sw,
                                 hipStream_t s) {
  const EngramWs w = engram_ws(workspace, N, d, M);
  return launch_engram_pass1(e, N, E, W, d, M, h, gamma_h, gamma_k, w.v, w.part_v, w.part_k,
                             f8, se, sw, s);
}

hipError_t launch_engram_gate(int64_t N, int64_t d, int64_t M, float eps, void* workspace,
                              hipStream_t s) {
  const EngramWs w = engram_ws(workspace, N, d, M);
  hipLaunchKernelGGL(engram_gate_kernel, dim3((unsigned)((N + kThreads - 1) / kThreads),
                                              (unsigned)M),
                     dim3(kThreads), 0, s, N, (int)d, (int)M, eps, w.part_v, w.part_k,
                     (int)(d / kColBlock), w.gate);
  return hipGetLastError();
}

hipError_t launch_engram_mix(int64_t B, int64_t T, int64_t d, int64_t M, const float* gamma_u,
                             const float* conv_w, int conv_k, int conv_dil, const void* h,
                             void* out, void* workspace, int add_resid, hipStream_t s) {
  const int64_t N = B * T;
  const EngramWs w = engram_ws(workspace, N, d, M);
  dim3 grid((unsigned)((T + kTB - 1) / kTB), (unsigned)B, (unsigned)((d + kCB - 1) / kCB));
  const int rowsL = kTB + (conv_k - 1) * conv_dil;
  const size_t lds = (size_t)rowsL * kCB * 2 + (size_t)2 * M * rowsL * 4;
  const auto* hh = static_cast<const uint16_t*>(h);
  auto* oo = static_cast<uint16_t*>(out);
#define PG_PASS2(KW)                                                                        \
  case KW:                                                                                  \
    if (M <= 4)                                                                             \
      hipLaunchKernelGGL((engram_pass2_kernel<KW, 4>), grid, dim3(kThreads), lds, s, T,     \
                         (int)d, (int)M, gamma_u, conv_w, conv_dil, w.v, w.gate, N, hh, oo, \
                         add_resid);                                                        \
    else                                                                                    \
      hipLaunchKernelGGL((engram_pass2_kernel<KW, kMaxBranches>), grid, dim3(kThreads), lds, \
                         s, T, (int)d, (int)M, gamma_u, conv_w, conv_dil, w.v, w.gate, N,   \
                         hh, oo, add_resid);                                                \
    break;
  switch (conv_k) {
    PG_PASS2(1) PG_PASS2(2) PG_PASS2(3) PG_PASS2(4) PG_PASS2(5) PG_PASS2(6) PG_PASS2(7)
    PG_PASS2(8)
    default:
      return hipErrorInvalidValue;
  }
#undef PG_PASS2
  return hipGetLastError();
}

hipError_t launch_engram(const void* e, int64_t B, int64_t T, int64_t E, const void* W,
                         int64_t d, int64_t M, float eps, const float* gamma_h,
                         const float* gamma_k, const float* gamma_u, const float* conv_w,
                         int conv_k, int conv_dil, const void* h, void* out,
                         void* workspace, int add_resid, int f8, int se, int sw,
                         hipStream_t s) {
  const int64_t N = B * T;
  hipError_t err = launch_engram_project(e, N, E, W, d, M, gamma_h, gamma_k, h, workspace, f8,
                                         se, sw, s);
  if (err != hipSuccess) return err;
  err = launch_engram_gate(N, d, M, eps, workspace, s);
  if (err != hipSuccess) return err;
  return launch_engram_mix(B, T, d, M, gamma_u, conv_w, conv_k, conv_dil, h, out, workspace,
                           add_resid, s);
}

}  // namespace pg
