// Internal declarations shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/pagegram.h"

namespace pg {

constexpr int kMaxOrders = PG_MAX_ORDERS;
constexpr int kMaxHeads = PG_MAX_HEADS;
constexpr int kMaxSignWords = 4;           // r <= 256
constexpr int kRoleStride = 5;             // c, a_0..a_3 (orders <= 4)
constexpr int kMaxRoles = kMaxOrders * (1 + kMaxHeads + kMaxHeads * kMaxSignWords);
constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

// Layout as the kernels see it (passed by value as a kernel argument). The
// host fills it from a validated pg_layout; magic[] holds floor((2^64-1)/P)
// for the exact 64-bit remainders below.
struct DevLayout {
  int32_t kind;       // pg_layout_kind
  int32_t n_min;
  int32_t O;          // number of orders
  int32_t K;
  int32_t r;
  int32_t W;          // sign words per head = ceil(r/64)
  int32_t use_signs;
  int32_t n_roles;    // O * (1 + K + K*W)
  uint64_t seed;
  uint64_t pad_id;
  uint64_t S, S_magic;
  int32_t S_pow2;     // S is a power of two: u mod S = u & (S - 1)
  int32_t pad1;
  int64_t n_rows;
  uint64_t P[kMaxOrders], P_magic[kMaxOrders];
  int64_t base[kMaxOrders];
  uint64_t Pk[kMaxOrders * kMaxHeads], Pk_magic[kMaxOrders * kMaxHeads];
  int64_t base_k[kMaxOrders * kMaxHeads];
};

// ---------------------------------------------------------------------------
// Integer helpers

// splitmix64 output function (Steele, Lea, Flood 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// x mod P with m = floor((2^64-1)/P): q = floor(x*m / 2^64) is the true
// quotient or one less (x*m/2^64 lies in (x/P - 1, x/P]), so one
// conditional subtraction finishes the remainder.
__device__ __forceinline__ uint64_t mod_magic(uint64_t x, uint64_t P, uint64_t m) {
  uint64_t q = __umul64hi(x, m);
  uint64_t rem = x - q * P;
  return rem >= P ? rem - P : rem;
}

// Constants of every hash role of the layout, into LDS: role q of order i
// is q_local = q - i*(1+K+K*W): 0 -> page hash, 1..K -> head hash k,
// then sign word (k, w). Slot 0 is the seed word c, slots 1..4 the odd
// multipliers a_j. Called by all threads of the block; ends with a barrier.
__device__ inline void load_role_consts(const DevLayout& L, uint64_t* rc) {
  const int R = 1 + L.K + L.K * L.W;
  const int total = L.n_roles * kRoleStride;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int slot = e % kRoleStride;
    const int q = e / kRoleStride;
    const int i = q / R;
    const int rr = q - i * R;
    const int n = L.n_min + i;
    int kind, k = 0, w = 0;
    if (rr == 0) {
      kind = 0;
    } else if (rr <= L.K) {
      kind = 1;
      k = rr - 1;
    } else {
      kind = 2;
      const int s = rr - 1 - L.K;
      k = s / L.W;
      w = s - k * L.W;
    }
    const uint64_t idx = (uint64_t)(((n * 4 + kind) * 64 + k) * 8 + w);
    uint64_t v = mix64(L.seed + (8 * idx + slot + 1) * kGolden);
    if (slot > 0) v |= 1ull;
    rc[e] = v;
  }
  __syncthreads();
}

// Canonical IDs are below 2^32, so each product is a 64 x 32-bit multiply.
__device__ __forceinline__ uint64_t role_hash(const uint64_t* rc, int q,
                                              const uint32_t* g, int n) {
  const uint64_t* c = rc + q * kRoleStride;
  uint64_t x = c[0];
  for (int j = 0; j < n; ++j) x ^= (uint64_t)g[j] * c[1 + j];
  return mix64(x);
}

// Canonical ID of token position t of a sequence starting at `seq`
// (pad_id when t < 0 or the token is outside [0, V)).
__device__ __forceinline__ uint32_t canon_at(const int32_t* __restrict__ seq,
                                             int64_t t, const int32_t* __restrict__ cmap,
                                             int64_t V, uint64_t pad) {
  if (t < 0) return (uint32_t)pad;
  const int32_t tok = seq[t];
  if (tok < 0 || (int64_t)tok >= V) return (uint32_t)pad;
  return (uint32_t)cmap[tok];
}

// Row of head k of order i for n-gram g (n = n_min + i), and the page for
// PageGram (-1 otherwise). rc holds the role constants.
__device__ __forceinline__ int64_t head_row(const DevLayout& L, const uint64_t* rc,
                                            const uint32_t* g, int i, int k,
                                            uint64_t* b_out, uint64_t* u_out,
                                            int64_t* page_out) {
  const int n = L.n_min + i;
  const int R = 1 + L.K + L.K * L.W;
  const uint64_t u = role_hash(rc, i * R + 1 + k, g, n);
  *u_out = u;
  if (L.kind == PG_PAGEGRAM) {
    const uint64_t b = role_hash(rc, i * R, g, n);
    const uint64_t p = mod_magic(b, L.P[i], L.P_magic[i]);
    const uint64_t slot = L.S_pow2 ? (u & (L.S - 1)) : mod_magic(u, L.S, L.S_magic);
    *b_out = b;
    *page_out = (int64_t)p;
    return L.base[i] + (int64_t)((p * (uint64_t)L.K + (uint64_t)k) * L.S + slot);
  }
  *b_out = role_hash(rc, i * R, g, n);
  *page_out = -1;
  const int hk = i * kMaxHeads + k;
  return L.base_k[hk] + (int64_t)mod_magic(u, L.Pk[hk], L.Pk_magic[hk]);
}

__device__ __forceinline__ uint64_t sign_word(const DevLayout& L, const uint64_t* rc,
                                              const uint32_t* g, int i, int k, int w) {
  if (!L.use_signs) return 0;
  const int R = 1 + L.K + L.K * L.W;
  return role_hash(rc, i * R + 1 + L.K + k * L.W + w, g, L.n_min + i);
}

// ---------------------------------------------------------------------------
// Float helpers

// Two fp32 values -> OCP E4M3 bytes (a in bits 0-7, b in bits 8-15). E4M3:
// sign, 4-bit exponent of bias 7, 3-bit mantissa, no infinities, 0x7F / 0xFF
// NaN, largest finite 448. Rounded to nearest, ties to the even mantissa;
// magnitudes >= 448 (infinities included) saturate to 448; NaN stays NaN
// with its sign; the sign of zero is kept. v_cvt_pk_fp8_f32 rounds to
// nearest even but turns overflow into NaN and NaN into 0xFF, so the values
// are clamped to +-448 first (v_med3) and NaN codes are set afterwards.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  const uint32_t na = 0x7Fu | ((__float_as_uint(a) >> 24) & 0x80u);
  const uint32_t nb = 0x7Fu | ((__float_as_uint(b) >> 24) & 0x80u);
  r = (a != a) ? ((r & 0xFF00u) | na) : r;
  r = (b != b) ? ((r & 0x00FFu) | (nb << 8)) : r;
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files; all return hipError_t)

hipError_t launch_index(const DevLayout& L, const int32_t* tokens, int64_t B, int64_t T,
                        const int32_t* cmap, int64_t V, int32_t* canon_out,
                        uint64_t* hash_out, int64_t* rows_out, int64_t* pages_out,
                        uint64_t* signs_out, int32_t* status, hipStream_t s);

hipError_t launch_gather(const DevLayout& L, int32_t table_dtype, const void* table,
                         const void* scales, const int64_t* rows, const uint64_t* signs,
                         int64_t n_tok, void* e_out, hipStream_t s);

// e_fp8: write e as E4M3(e 2^e_scale_exp) bytes instead of bf16 / fp32.
hipError_t launch_index_gather(const DevLayout& L, int32_t table_dtype, const void* table,
                               const void* scales, const int32_t* tokens, int64_t B,
                               int64_t T, const int32_t* cmap, int64_t V, void* e_out,
                               int32_t* status, int e_fp8, int e_scale_exp, hipStream_t s);

// dst[i] = E4M3(src[i] 2^scale_exp) for bf16 or fp32 src.
hipError_t launch_quantize_fp8(const void* src, int32_t src_dtype, int64_t n, int scale_exp,
                               uint8_t* dst, hipStream_t s);

// Scalar-gate projection: out[N][d] = resid + g * e W^T.
hipError_t launch_project_scalar(int32_t dtype, const void* e, int64_t N, int64_t E,
                                 const void* W, int64_t d, float g, const void* resid,
                                 void* out, hipStream_t s);

// pg_forward's fused path for bf16 tables of 64-element rows under the
// scalar gate. launch_records writes, for head slot hs = i K + k and token
// t, rec[hs][t] = {row, the sign bits of the two MFMA lane halves, 0}
// (4 x uint32; B T (O K) 16 bytes); launch_project_gathered is the
// scalar-gate projection with its E operand (E = 64 O K) gathered from the
// table by those records.
hipError_t launch_records(const DevLayout& L, const int32_t* tokens, int64_t B, int64_t T,
                          const int32_t* cmap, int64_t V, void* rec, int32_t* status,
                          hipStream_t s);
hipError_t launch_project_gathered(const void* table, const void* rec, int64_t N, int64_t E,
                                  const void* W, int64_t d, float g, const void* resid,
                                  void* out, hipStream_t s);

// The same on E4M3 operands e8 = E4M3(e 2^se), W8 = E4M3(W 2^sw).
hipError_t launch_project_scalar_fp8(const void* e8, int64_t N, int64_t E, const void* W8,
                                     int64_t d, float g, const void* resid, void* out,
                                     int se, int sw, hipStream_t s);

// fp32-output GEMM with optional split K (partials at out + s * M * ldo).
// Engram pass 1 through the slot-ring kernel (gemm_slots.hip): bf16
// operands (E a multiple of 64) or, with f8, E4M3 ones with scales 2^se
// (e) and 2^sw (W) (E a multiple of 128); d a multiple of 256 (checked by
// the caller).
hipError_t launch_engram_pass1_slots(const void* e, int64_t N, int64_t E, const void* W,
                                     int64_t d, int64_t Mbr, const void* h,
                                     const float* gamma_h, const float* gamma_k, uint16_t* v,
                                     float* part_v, float* part_k, int f8, int se, int sw,
                                     hipStream_t s);
hipError_t launch_gemm_f32(const void* A, int lda, const void* B, int ldb, int64_t M, int N,
                           int Kc, int splits, float g, float* out, int64_t ldo,
                           hipStream_t s);

// Backward pass of the scalar gate and the sparse table update
// (backward.hip): workspace geometry, then the launchers.
struct BackwardPlan {
  int splits;       // K splits of the dW GEMM
  int kc;           // tokens per split (multiple of 64)
  int64_t kpad;     // splits * kc: padded token count of the transposes
  int64_t nblk;     // blocks of the sort / segment kernels
  int64_t off_dyT, off_eT, off_WT, off_part, off_k0, off_k1, off_v0, off_v1, off_counts,
      off_flags, off_seg, off_long;
  int64_t bytes;
};
BackwardPlan backward_plan(int64_t N, int64_t d, int64_t E, int64_t L);
hipError_t launch_backward_scalar(const DevLayout& L, const BackwardPlan& p, float g,
                                  const int64_t* rows, const uint64_t* signs, const void* e,
                                  const void* dy, const void* W, int64_t N, int64_t d,
                                  float* dW, float* de, int64_t* urows, float* ugrad,
                                  int64_t* n_unique, void* workspace, hipStream_t s);
hipError_t launch_set_i64(int64_t* p, int64_t v, hipStream_t s);
hipError_t launch_rms_step(const int64_t* urows, const float* ugrad, const int64_t* n_unique,
                           int64_t max_unique, int r, float* table, float* vhat, int64_t* last,
                           int64_t step, float lr, float beta2, float wd, float eps,
                           hipStream_t s);
hipError_t launch_rms_flush(int64_t R, int r, float* table, float* vhat, int64_t* last,
                            int64_t step, float lr, float beta2, float wd, hipStream_t s);

// Staging of table units into an HBM cache (stage.hip): workspace geometry
// for n_tok tokens with units of U rows, then the launcher. rb: bytes of a
// row in the data array (NF4: the r/2 code bytes; scales are separate).
struct StagePlan {
  int U;
  int share;        // the K heads of a token-order share a unit (PageGram pages)
  int64_t n_look, max_units, H, nb;
  int64_t off_keys, off_ranks, off_bcount, off_ufirst, off_ucount;
  int64_t bytes;
};
StagePlan stage_plan(const DevLayout& L, int U, int share, int64_t n_tok);
hipError_t launch_stage(const DevLayout& L, const StagePlan& p, int rb, const void* src,
                        const void* src_scales, const int64_t* rows, void* dst,
                        void* dst_scales, int64_t* cache_rows, int64_t* n_units,
                        int64_t* ufirst_out, void* workspace, hipStream_t s);

// Engram fusion (bf16 or, with f8, E4M3 operands of scales se, sw): workspace
// layout described in engram_workspace_bytes.
int64_t engram_workspace_bytes(int64_t N, int64_t d, int64_t M);
hipError_t launch_engram_pass1(const void* e, int64_t N, int64_t E, const void* W,
                               int64_t d, int64_t Mbr, const void* h,
                               const float* gamma_h, const float* gamma_k, uint16_t* v,
                               float* part_v, float* part_k, int f8, int se, int sw,
                               hipStream_t s);
// The three stages launch_engram runs: pass 1 (v and the partial sums),
// the per-token gate, pass 2 (conv, SiLU, residual).
hipError_t launch_engram_project(const void* e, int64_t N, int64_t E, const void* W, int64_t d,
                                 int64_t M, const float* gamma_h, const float* gamma_k,
                                 const void* h, void* workspace, int f8, int se, int sw,
                                 hipStream_t s);
hipError_t launch_engram_gate(int64_t N, int64_t d, int64_t M, float eps, void* workspace,
                              hipStream_t s);
hipError_t launch_engram_mix(int64_t B, int64_t T, int64_t d, int64_t M, const float* gamma_u,
                             const float* conv_w, int conv_k, int conv_dil, const void* h,
                             void* out, void* workspace, int add_resid, hipStream_t s);
hipError_t launch_engram(const void* e, int64_t B, int64_t T, int64_t E, const void* W,
                         int64_t d, int64_t M, float eps, const float* gamma_h,
                         const float* gamma_k, const float* gamma_u, const float* conv_w,
                         int conv_k, int conv_dil, const void* h, void* out,
                         void* workspace, int add_resid, int f8, int se, int sw,
                         hipStream_t s);

// Streaming read of bytes (a multiple of 16) at src by `blocks` blocks; one
// word per block into sink (probe.hip).
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, int blocks,
                             hipStream_t s);

}  // namespace pg
