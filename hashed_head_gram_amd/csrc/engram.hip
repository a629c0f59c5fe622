// Engram fusion, pass 2 (gfx950), after the projection GEMM's pass 1.
//
// Engram notes §3.3-3.4 with M branches sharing v = W_V e:
//   alpha^m_t = sigmoid(RMSNorm_h(h^m_t) . RMSNorm_k(k^m_t) / sqrt(d))
//   u^m_t     = alpha^m_t v_t
//   z^m_t     = RMSNorm_u(u^m_t) = gamma_u * v_t * alpha / sqrt(alpha^2 ms(v_t) + eps)
//   out^m_t   = h^m_t + u^m_t + SiLU(sum_j w_j * z^m_{t-(kw-1-j)*dil})
// From pass 1 the workspace holds v (bf16) and per-token partial sums over
// 128-column blocks: sum v^2, and per branch sum k^2, sum gamma_h gamma_k h k,
// sum h^2. RMSNorm_h(h).RMSNorm_k(k) = that dot / (rms(h) rms(k)).
//
// A block takes TB tokens of one sequence and 256 channels. It first turns
// the partial sums into (alpha, z-scale) per token and branch for its tokens
// and the (kw-1)*dil tokens before them, stages that v window in LDS, then
// each lane produces 8 channels of one token for all branches with 16-byte
// loads of h and stores of out.
#include "common.h"

namespace pg {

hipError_t launch_engram_pass1(const void* e, int64_t N, int64_t E, const void* W,
                               int64_t d, int64_t Mbr, const void* h,
                               const float* gamma_h, const float* gamma_k, uint16_t* v,
                               float* part_v, float* part_k, hipStream_t s);

namespace {

constexpr int kThreads = 256;
constexpr int kTB = 32;          // tokens per block
constexpr int kCB = 256;         // channels per block
constexpr int kMaxHalo = 64;     // (conv_k - 1) * conv_dil
constexpr int kMaxBr = 8;
constexpr int kMaxTaps = 8;
constexpr int kColBlock = 128;   // pass-1 column block of the partial sums

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

__global__ __launch_bounds__(kThreads) void engram_pass2_kernel(
    int64_t T, int d, int Mbr, float eps, const float* __restrict__ gamma_u,
    const float* __restrict__ conv_w, int kw, int dil, const uint16_t* __restrict__ v,
    const float* __restrict__ part_v, const float* __restrict__ part_k, int n_cb,
    int64_t N, const uint16_t* __restrict__ h, uint16_t* __restrict__ out, int add_resid) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[(kTB + kMaxHalo) * kCB];
  __shared__ float alphaL[kMaxBr][kTB + kMaxHalo];
  __shared__ float facL[kMaxBr][kTB + kMaxHalo];

  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kTB;
  const int c0 = blockIdx.z * kCB;
  const int H = (kw - 1) * dil;
  const int rowsL = kTB + H;
  const int tid = threadIdx.x;
  const float inv_d = 1.0f / (float)d;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);

  // Per-token scalars for positions t0-H .. t0+TB-1 (LDS index tau - (t0-H)).
  for (int q = tid; q < rowsL * Mbr; q += kThreads) {
    const int m = q / rowsL;
    const int tl = q - m * rowsL;
    const int64_t tau = t0 - H + tl;
    float alpha = 0.f, fac = 0.f;
    if (tau >= 0 && tau < T) {
      const int64_t tok = b * T + tau;
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
      const float zlogit = dot * rh * rk * inv_sqrt_d;
      alpha = 1.0f / (1.0f + expf(-zlogit));
      fac = alpha / sqrtf(alpha * alpha * (sv * inv_d) + eps);
    }
    alphaL[m][tl] = alpha;
    facL[m][tl] = fac;
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
  float w[8][kMaxTaps];
  float gu[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    gu[x] = gamma_u[c + x];
#pragma unroll
    for (int j = 0; j < kMaxTaps; ++j) w[x][j] = j < kw ? conv_w[(c + x) * kw + j] : 0.f;
  }
  for (int tl = tid >> 5; tl < kTB; tl += kThreads / 32) {
    const int64_t t = t0 + tl;
    if (t >= T) break;
    const int li = tl + H;  // LDS index of t
    float vc[8];
    {
      const uint4 raw = *reinterpret_cast<const uint4*>(&vt[li * kCB + cg * 8]);
      const uint32_t ws[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        vc[2 * x] = bf16_to_f32((uint16_t)(ws[x] & 0xFFFFu));
        vc[2 * x + 1] = bf16_to_f32((uint16_t)(ws[x] >> 16));
      }
    }
    for (int m = 0; m < Mbr; ++m) {
      float conv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < kw; ++j) {
        const int lj = li - (kw - 1 - j) * dil;   // >= 0; zero rows before the start
        const float f = facL[m][lj];
        const uint4 raw = *reinterpret_cast<const uint4*>(&vt[lj * kCB + cg * 8]);
        const uint32_t ws[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          conv[2 * x] += w[2 * x][j] * (gu[2 * x] * bf16_to_f32((uint16_t)(ws[x] & 0xFFFFu)) * f);
          conv[2 * x + 1] +=
              w[2 * x + 1][j] * (gu[2 * x + 1] * bf16_to_f32((uint16_t)(ws[x] >> 16)) * f);
        }
      }
      const float alpha = alphaL[m][li];
      const int64_t o = ((int64_t)m * N + b * T + t) * d + c;
      float hv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (add_resid) {
        const uint4 raw = *reinterpret_cast<const uint4*>(h + o);
        const uint32_t ws[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          hv[2 * x] = bf16_to_f32((uint16_t)(ws[x] & 0xFFFFu));
          hv[2 * x + 1] = bf16_to_f32((uint16_t)(ws[x] >> 16));
        }
      }
      uint32_t res[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        float y0 = conv[2 * x], y1 = conv[2 * x + 1];
        y0 = y0 / (1.0f + expf(-y0));
        y1 = y1 / (1.0f + expf(-y1));
        const float o0 = hv[2 * x] + (alpha * vc[2 * x] + y0);
        const float o1 = hv[2 * x + 1] + (alpha * vc[2 * x + 1] + y1);
        res[x] = (uint32_t)f32_to_bf16(o0) | ((uint32_t)f32_to_bf16(o1) << 16);
      }
      *reinterpret_cast<uint4*>(out + o) = make_uint4(res[0], res[1], res[2], res[3]);
    }
  }
}

}  // namespace

int64_t engram_workspace_bytes(int64_t N, int64_t d, int64_t M) {
  const int64_t n_cb = d / kColBlock;
  return align256(N * d * 2) + align256(n_cb * N * 4) + align256(M * 3 * n_cb * N * 4);
}

hipError_t launch_engram(const void* e, int64_t B, int64_t T, int64_t E, const void* W,
                         int64_t d, int64_t M, float eps, const float* gamma_h,
                         const float* gamma_k, const float* gamma_u, const float* conv_w,
                         int conv_k, int conv_dil, const void* h, void* out,
                         void* workspace, int add_resid, hipStream_t s) {
  const int64_t N = B * T;
  const int64_t n_cb = d / kColBlock;
  auto* base = static_cast<uint8_t*>(workspace);
  auto* v = reinterpret_cast<uint16_t*>(base);
  auto* part_v = reinterpret_cast<float*>(base + align256(N * d * 2));
  auto* part_k = reinterpret_cast<float*>(base + align256(N * d * 2) + align256(n_cb * N * 4));
  hipError_t err = launch_engram_pass1(e, N, E, W, d, M, h, gamma_h, gamma_k, v, part_v,
                                       part_k, s);
  if (err != hipSuccess) return err;
  dim3 grid((unsigned)((T + kTB - 1) / kTB), (unsigned)B, (unsigned)((d + kCB - 1) / kCB));
  hipLaunchKernelGGL(engram_pass2_kernel, grid, dim3(kThreads), 0, s, T, (int)d, (int)M, eps,
                     gamma_u, conv_w, conv_k, conv_dil, v, part_v, part_k, (int)n_cb, N,
                     static_cast<const uint16_t*>(h), static_cast<uint16_t*>(out), add_resid);
  return hipGetLastError();
}

}  // namespace pg
