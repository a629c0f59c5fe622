// C ABI entry points: argument validation, layout preparation, dispatch.
// Every check that can fail runs before anything is enqueued.
#include <limits.h>

#include <mutex>

#include "common.h"

namespace {

using pg::DevLayout;

constexpr int64_t kMaxTokens = (int64_t)1 << 31;
constexpr int kReadProbeBlocks = 4096;   // pg_read_probe's grid (one sink word each)
constexpr int64_t kRowLimit = (int64_t)1 << 62;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Validate a pg_layout and fill the kernels' view of it.
int prepare_layout(const pg_layout* in, DevLayout* L) {
  if (!in) return PG_EINVAL;
  if (in->kind != PG_PAGEGRAM && in->kind != PG_ENGRAM) return PG_EINVAL;
  if (in->n_min < 1 || in->n_max < in->n_min || in->n_max > PG_MAX_ORDERS) return PG_EINVAL;
  if (in->K < 1 || in->K > PG_MAX_HEADS) return PG_EINVAL;
  if (in->r < 1 || in->r > 64 * pg::kMaxSignWords) return PG_EINVAL;
  if (in->pad_id < 0) return PG_EINVAL;
  if (in->use_signs != 0 && in->use_signs != 1) return PG_EINVAL;
  *L = DevLayout{};
  L->kind = in->kind;
  L->n_min = in->n_min;
  L->O = in->n_max - in->n_min + 1;
  L->K = in->K;
  L->r = in->r;
  L->W = (in->r + 63) / 64;
  L->use_signs = in->use_signs;
  L->n_roles = L->O * (1 + L->K + L->K * L->W);
  L->seed = in->hash_seed;
  L->pad_id = (uint64_t)(uint32_t)in->pad_id;
  int64_t acc = 0;
  if (in->kind == PG_PAGEGRAM) {
    if (in->S < 1) return PG_EINVAL;
    L->S = (uint64_t)in->S;
    L->S_magic = UINT64_MAX / L->S;
    L->S_pow2 = (L->S & (L->S - 1)) == 0;
    const int64_t per_page = (int64_t)in->K * in->S;
    for (int i = 0; i < L->O; ++i) {
      const int64_t P = in->pages[i];
      if (P < 1) return PG_EINVAL;
      if (P > (kRowLimit - acc) / per_page) return PG_ERANGE;
      L->P[i] = (uint64_t)P;
      L->P_magic[i] = UINT64_MAX / (uint64_t)P;
      L->base[i] = acc;
      acc += P * per_page;
    }
  } else {
    L->S = 1;
    L->S_magic = UINT64_MAX;
    L->S_pow2 = 1;
    for (int i = 0; i < L->O; ++i)
      for (int k = 0; k < L->K; ++k) {
        const int64_t P = in->head_rows[i][k];
        if (P < 1) return PG_EINVAL;
        if (P > kRowLimit - acc) return PG_ERANGE;
        const int hk = i * pg::kMaxHeads + k;
        L->Pk[hk] = (uint64_t)P;
        L->Pk_magic[hk] = UINT64_MAX / (uint64_t)P;
        L->base_k[hk] = acc;
        acc += P;
      }
  }
  L->n_rows = acc;
  return PG_OK;
}

int table_e_dtype(int32_t table_dtype) { return table_dtype == PG_F32 ? PG_F32 : PG_BF16; }

int check_table(const DevLayout& L, const pg_table* t) {
  if (!t || !t->data) return PG_EINVAL;
  if (!aligned(t->data, 16)) return PG_EINVAL;
  if (t->n_rows != L.n_rows) return PG_EINVAL;
  switch (t->dtype) {
    case PG_F32:
      if (L.r % 4) return PG_EUNSUPPORTED;
      break;
    case PG_BF16:
      if (L.r % 8) return PG_EUNSUPPORTED;
      break;
    case PG_NF4:
      if (L.r % 32) return PG_EUNSUPPORTED;
      if (!t->scales || !aligned(t->scales, 2)) return PG_EINVAL;
      break;
    default:
      return PG_EINVAL;
  }
  return PG_OK;
}

int check_tokens(const int32_t* tokens, int64_t B, int64_t T, const int32_t* cmap, int64_t V) {
  if (B < 0 || T < 0) return PG_EINVAL;
  if (T > 0 && B > kMaxTokens / T) return PG_ERANGE;
  if (B * T == 0) return PG_OK;
  if (!tokens || !cmap || V < 1) return PG_EINVAL;
  return PG_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PG_OK : PG_EHIP; }

int check_fuse(const pg_fuse* f, int64_t B, int64_t T, int64_t e_dim) {
  if (!f) return PG_EINVAL;
  if (f->gate != PG_GATE_SCALAR && f->gate != PG_GATE_ENGRAM) return PG_EINVAL;
  if (f->dtype != PG_F32 && f->dtype != PG_BF16) return PG_EINVAL;
  if (f->d < 1 || e_dim < 1) return PG_EINVAL;
  if (B < 0 || T < 0) return PG_EINVAL;
  if (T > 0 && B > kMaxTokens / T) return PG_ERANGE;
  if (e_dim > INT_MAX) return PG_ERANGE;
  if (f->increment_only != 0 && f->increment_only != 1) return PG_EINVAL;
  if (f->dtype == PG_BF16 && e_dim % 8) return PG_EUNSUPPORTED;
  if (f->dtype == PG_F32 && e_dim % 4) return PG_EUNSUPPORTED;
  if (f->gate == PG_GATE_ENGRAM) {
    if (f->dtype != PG_BF16) return PG_EUNSUPPORTED;
    if (f->d % 256 || e_dim % 64) return PG_EUNSUPPORTED;
    if (f->M < 1 || f->M > 8) return PG_EINVAL;
    if (f->conv_k < 1 || f->conv_k > 8 || f->conv_dil < 1) return PG_EINVAL;
    if ((int64_t)(f->conv_k - 1) * f->conv_dil > 64) return PG_EUNSUPPORTED;
    if (!f->gamma_h || !f->gamma_k || !f->gamma_u || !f->conv_w) return PG_EINVAL;
    if (!(f->eps >= 0.0f)) return PG_EINVAL;
    if (B > 65535) return PG_EUNSUPPORTED;
    if ((int64_t)(1 + f->M) * f->d > INT_MAX) return PG_ERANGE;
  }
  return PG_OK;
}

int64_t project_workspace(const pg_fuse* f, int64_t N) {
  if (f->gate == PG_GATE_ENGRAM) return pg::engram_workspace_bytes(N, f->d, f->M);
  return 0;
}

int64_t elt_bytes(int32_t dt) { return dt == PG_F32 ? 4 : 2; }

// Records of the gathered projection: 64-element rows (one sign word per
// head), 32-bit record offsets within a head slot.
constexpr int64_t kMaxRecordTokens = (int64_t)1 << 28;
bool records_ok(const DevLayout& L, int64_t N) {
  return L.r == 64 && L.W == 1 && N <= kMaxRecordTokens;
}

// The gathered projection: bf16 tables of 64-element rows whose byte
// offsets fit 32 bits, under the scalar gate.
bool gathered_ok(const DevLayout& L, const pg_table* t, const pg_fuse* f, int64_t N) {
  return records_ok(L, N) && t->dtype == PG_BF16 && f->gate == PG_GATE_SCALAR &&
         L.n_rows <= ((int64_t)1 << 25);
}

// Projection + fusion on an e already in device memory.
int run_project(const pg_fuse* f, const void* e, int64_t B, int64_t T, int64_t e_dim,
                const void* W, const void* resid, void* out, void* ws, hipStream_t s) {
  const int64_t N = B * T;
  if (f->gate == PG_GATE_SCALAR) {
    const void* x = f->increment_only ? nullptr : resid;
    return hip_status(pg::launch_project_scalar(f->dtype, e, N, e_dim, W, f->d, f->g, x, out, s));
  }
  return hip_status(pg::launch_engram(e, B, T, e_dim, W, f->d, f->M, f->eps, f->gamma_h,
                                      f->gamma_k, f->gamma_u, f->conv_w, f->conv_k,
                                      f->conv_dil, resid, out, ws, f->increment_only ? 0 : 1,
                                      0, 0, 0, s));
}

// FP8 operands: scale exponents within +-64, e_dim a multiple of 128 (the
// FP8 MFMA's K stage), bf16 residual and output.
constexpr int kMaxScaleExp = 64;
bool scale_ok(int32_t se) { return se >= -kMaxScaleExp && se <= kMaxScaleExp; }

int check_fp8_fuse(const pg_fuse* f, int64_t B, int64_t T, int64_t e_dim, int32_t se,
                   int32_t sw) {
  const int st = check_fuse(f, B, T, e_dim);
  if (st != PG_OK) return st;
  if (!scale_ok(se) || !scale_ok(sw)) return PG_EINVAL;
  if (f->dtype != PG_BF16) return PG_EUNSUPPORTED;
  if (e_dim % 128) return PG_EUNSUPPORTED;
  return PG_OK;
}

int run_project_fp8(const pg_fuse* f, const void* e8, int64_t B, int64_t T, int64_t e_dim,
                    const void* W8, int32_t se, int32_t sw, const void* resid, void* out,
                    void* ws, hipStream_t s) {
  const int64_t N = B * T;
  if (f->gate == PG_GATE_SCALAR) {
    const void* x = f->increment_only ? nullptr : resid;
    return hip_status(
        pg::launch_project_scalar_fp8(e8, N, e_dim, W8, f->d, f->g, x, out, se, sw, s));
  }
  return hip_status(pg::launch_engram(e8, B, T, e_dim, W8, f->d, f->M, f->eps, f->gamma_h,
                                      f->gamma_k, f->gamma_u, f->conv_w, f->conv_k,
                                      f->conv_dil, resid, out, ws, f->increment_only ? 0 : 1,
                                      1, se, sw, s));
}

}  // namespace

extern "C" {

PG_API const char* pg_strerror(int status) {
  switch (status) {
    case PG_OK: return "ok";
    case PG_EINVAL: return "invalid argument (NULL pointer, size, alignment or layout)";
    case PG_EUNSUPPORTED: return "unsupported shape or dtype combination";
    case PG_EHIP: return "HIP launch or runtime error";
    case PG_ERANGE: return "size out of range";
    default: return "unknown status";
  }
}

PG_API uint32_t pg_hash_version(void) { return 1u; }

PG_API int pg_layout_rows(const pg_layout* layout, int64_t* n_rows) {
  if (!n_rows) return PG_EINVAL;
  DevLayout L;
  const int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  *n_rows = L.n_rows;
  return PG_OK;
}

PG_API int64_t pg_workspace_size(const pg_layout* layout, const pg_fuse* fuse, int64_t B,
                                 int64_t T) {
  if (!fuse || B < 0 || T < 0) return PG_EINVAL;
  if (T > 0 && B > kMaxTokens / T) return PG_ERANGE;
  const int64_t N = B * T;
  int64_t bytes = 0;
  if (layout) {
    DevLayout L;
    const int st = prepare_layout(layout, &L);
    if (st != PG_OK) return st;
    bytes += align256(N * (int64_t)L.O * L.K * L.r * elt_bytes(fuse->dtype));
  }
  if (fuse->gate == PG_GATE_ENGRAM) {
    if (fuse->d < 1 || fuse->M < 1 || fuse->M > 8) return PG_EINVAL;
  }
  return bytes + project_workspace(fuse, N);
}

PG_API int pg_index(const pg_layout* layout, const int32_t* tokens, int64_t B, int64_t T,
                    const int32_t* canon_map, int64_t V, int32_t* canon_out,
                    uint64_t* hash_out, int64_t* rows_out, int64_t* pages_out,
                    uint64_t* signs_out, int32_t* dev_status, hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_tokens(tokens, B, T, canon_map, V);
  if (st != PG_OK) return st;
  if (B * T == 0) return PG_OK;
  if (!rows_out || !signs_out) return PG_EINVAL;
  return hip_status(pg::launch_index(L, tokens, B, T, canon_map, V, canon_out, hash_out,
                                     rows_out, pages_out, signs_out, dev_status, stream));
}

PG_API int pg_gather(const pg_layout* layout, const pg_table* table, const int64_t* rows,
                     const uint64_t* signs, int64_t n_tok, int32_t e_dtype, void* e_out,
                     hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_table(L, table);
  if (st != PG_OK) return st;
  if (n_tok < 0) return PG_EINVAL;
  if (n_tok > kMaxTokens) return PG_ERANGE;
  if (e_dtype != table_e_dtype(table->dtype)) return PG_EUNSUPPORTED;
  if (n_tok == 0) return PG_OK;
  if (!rows || !e_out || !aligned(e_out, 16)) return PG_EINVAL;
  if (!signs && L.use_signs) return PG_EINVAL;
  return hip_status(pg::launch_gather(L, table->dtype, table->data, table->scales, rows,
                                      signs, n_tok, e_out, stream));
}

PG_API int pg_index_gather(const pg_layout* layout, const pg_table* table,
                           const int32_t* tokens, int64_t B, int64_t T,
                           const int32_t* canon_map, int64_t V, int32_t e_dtype,
                           void* e_out, int32_t* dev_status, hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_table(L, table);
  if (st != PG_OK) return st;
  st = check_tokens(tokens, B, T, canon_map, V);
  if (st != PG_OK) return st;
  if (e_dtype != table_e_dtype(table->dtype)) return PG_EUNSUPPORTED;
  if (B * T == 0) return PG_OK;
  if (!e_out || !aligned(e_out, 16)) return PG_EINVAL;
  return hip_status(pg::launch_index_gather(L, table->dtype, table->data, table->scales,
                                            tokens, B, T, canon_map, V, e_out, dev_status, 0, 0,
                                            stream));
}

PG_API int pg_project_gate(const pg_fuse* fuse, const void* e, int64_t B, int64_t T,
                           int64_t e_dim, const void* W, const void* resid, void* out,
                           void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  int st = check_fuse(fuse, B, T, e_dim);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!e || !W || !out) return PG_EINVAL;
  if (!aligned(e, 16) || !aligned(W, 16) || !aligned(out, 16)) return PG_EINVAL;
  if (resid && !aligned(resid, 16)) return PG_EINVAL;
  if (fuse->gate == PG_GATE_ENGRAM && !resid) return PG_EINVAL;
  const int64_t need = project_workspace(fuse, N);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return PG_EINVAL;
  return run_project(fuse, e, B, T, e_dim, W, resid, out, workspace, stream);
}

namespace {

// pg_forward's validation and dispatch; `ws == nullptr` with
// use_scratch set takes the workspace from the device's scratch array.
int forward_impl(const pg_layout* layout, const pg_table* table, const pg_fuse* fuse,
                 const int32_t* tokens, int64_t B, int64_t T, const int32_t* canon_map,
                 int64_t V, const void* W, const void* resid, void* out, void* workspace,
                 int64_t workspace_bytes, bool use_scratch, int32_t* dev_status,
                 hipStream_t stream);

}  // namespace

PG_API int pg_forward(const pg_layout* layout, const pg_table* table, const pg_fuse* fuse,
                      const int32_t* tokens, int64_t B, int64_t T, const int32_t* canon_map,
                      int64_t V, const void* W, const void* resid, void* out,
                      void* workspace, int64_t workspace_bytes, int32_t* dev_status,
                      hipStream_t stream) {
  return forward_impl(layout, table, fuse, tokens, B, T, canon_map, V, W, resid, out,
                      workspace, workspace_bytes, false, dev_status, stream);
}

// ---------------------------------------------------------------------------
// pg_forward_noalloc: pg_forward with its workspace in a file-scope device
// array, for callers that cannot allocate device memory. Each GPU the
// library runs on holds one copy of the array (PG_NOALLOC_SCRATCH_BYTES)
// from the code object's load until the process ends; its device address
// is looked up once per device and kept. Calls on one GPU share the array,
// so calls that overlap on one GPU (different streams, different threads)
// race on it. No kernel of the path relies on the workspace starting at
// zero (every byte a kernel reads was written earlier in the same call), so
// nothing is cleared.

static __device__ __align__(256) uint8_t scratch[PG_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];   // per device ordinal; null until looked up

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream); the lookup runs once per device, with that
// device current.
int scratch_for(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return PG_EHIP;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return PG_EHIP;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return PG_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return PG_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return PG_EHIP;
    if (e != hipSuccess || !p) return PG_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PG_OK;
}

int forward_impl(const pg_layout* layout, const pg_table* table, const pg_fuse* fuse,
                 const int32_t* tokens, int64_t B, int64_t T, const int32_t* canon_map,
                 int64_t V, const void* W, const void* resid, void* out, void* workspace,
                 int64_t workspace_bytes, bool use_scratch, int32_t* dev_status,
                 hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_table(L, table);
  if (st != PG_OK) return st;
  st = check_tokens(tokens, B, T, canon_map, V);
  if (st != PG_OK) return st;
  const int64_t e_dim = (int64_t)L.O * L.K * L.r;
  st = check_fuse(fuse, B, T, e_dim);
  if (st != PG_OK) return st;
  if (fuse->dtype != table_e_dtype(table->dtype)) return PG_EUNSUPPORTED;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!W || !out || !aligned(W, 16) || !aligned(out, 16)) return PG_EINVAL;
  if (resid && !aligned(resid, 16)) return PG_EINVAL;
  if (fuse->gate == PG_GATE_ENGRAM && !resid) return PG_EINVAL;
  const int64_t e_bytes = align256(N * e_dim * elt_bytes(fuse->dtype));
  const int64_t need = e_bytes + project_workspace(fuse, N);
  if (use_scratch) {
    if (need > PG_NOALLOC_SCRATCH_BYTES) return PG_ERANGE;
    st = scratch_for(stream, &workspace);
    if (st != PG_OK) return st;
    workspace_bytes = PG_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return PG_EINVAL;
  // bf16 table rows of 64 elements under the scalar gate: the projection
  // gathers its E operand from the table itself, by per-(head slot, token)
  // records of row and signs (same products, same order); the records take
  // N (O K) 16 bytes of the workspace
  if (gathered_ok(L, table, fuse, N)) {
    const void* x = fuse->increment_only ? nullptr : resid;
    st = hip_status(pg::launch_records(L, tokens, B, T, canon_map, V, workspace, dev_status,
                                       stream));
    if (st != PG_OK) return st;
    return hip_status(pg::launch_project_gathered(table->data, workspace, N, e_dim, W, fuse->d,
                                                  fuse->g, x, out, stream));
  }
  void* e = workspace;
  void* ws = static_cast<uint8_t*>(workspace) + e_bytes;
  st = hip_status(pg::launch_index_gather(L, table->dtype, table->data, table->scales, tokens,
                                          B, T, canon_map, V, e, dev_status, 0, 0, stream));
  if (st != PG_OK) return st;
  return run_project(fuse, e, B, T, e_dim, W, resid, out, ws, stream);
}

}  // namespace

PG_API int pg_forward_noalloc(const pg_layout* layout, const pg_table* table,
                              const pg_fuse* fuse, const int32_t* tokens, int64_t B, int64_t T,
                              const int32_t* canon_map, int64_t V, const void* W,
                              const void* resid, void* out, int32_t* dev_status,
                              hipStream_t stream) {
  return forward_impl(layout, table, fuse, tokens, B, T, canon_map, V, W, resid, out, nullptr,
                      0, true, dev_status, stream);
}

PG_API int pg_index_records(const pg_layout* layout, const int32_t* tokens, int64_t B,
                            int64_t T, const int32_t* canon_map, int64_t V, void* rec_out,
                            int32_t* dev_status, hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_tokens(tokens, B, T, canon_map, V);
  if (st != PG_OK) return st;
  if (!records_ok(L, B * T)) return L.r != 64 ? PG_EUNSUPPORTED : PG_ERANGE;
  if (B * T == 0) return PG_OK;
  if (!rec_out || !aligned(rec_out, 16)) return PG_EINVAL;
  return hip_status(pg::launch_records(L, tokens, B, T, canon_map, V, rec_out, dev_status,
                                       stream));
}

PG_API int pg_project_gathered(const pg_layout* layout, const pg_table* table,
                               const pg_fuse* fuse, const void* rec, int64_t B, int64_t T,
                               const void* W, const void* resid, void* out,
                               hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_table(L, table);
  if (st != PG_OK) return st;
  const int64_t e_dim = (int64_t)L.O * L.K * L.r;
  st = check_fuse(fuse, B, T, e_dim);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (fuse->dtype != PG_BF16 || !gathered_ok(L, table, fuse, N)) return PG_EUNSUPPORTED;
  if (N == 0) return PG_OK;
  if (!rec || !W || !out || !aligned(rec, 16) || !aligned(W, 16) || !aligned(out, 16))
    return PG_EINVAL;
  if (resid && !aligned(resid, 16)) return PG_EINVAL;
  const void* x = fuse->increment_only ? nullptr : resid;
  return hip_status(pg::launch_project_gathered(table->data, rec, N, e_dim, W, fuse->d, fuse->g,
                                                x, out, stream));
}

// ---------------------------------------------------------------------------
// Staging from a host-resident table

namespace {

// Rows per staging unit: a PageGram page, or the Engram-style tables'
// 4 KiB run (row bytes: fp32 4r, bf16 2r, NF4 r/2 codes + 2 scale bytes).
int64_t stage_unit_rows(const DevLayout& L, int32_t dt, int32_t unit_kind) {
  if (unit_kind == PG_STAGE_ROW) return 1;
  if (L.kind == PG_PAGEGRAM) return (int64_t)L.K * (int64_t)L.S;
  const int64_t rb = dt == PG_F32 ? 4 * L.r : dt == PG_BF16 ? 2 * L.r : L.r / 2 + 2;
  const int64_t u = 4096 / rb;
  return u < 1 ? 1 : u;
}

int stage_share(const DevLayout& L, int32_t unit_kind) {
  return L.kind == PG_PAGEGRAM && unit_kind == PG_STAGE_PAGE ? 1 : 0;
}

int64_t data_row_bytes(const DevLayout& L, int32_t dt) {
  return dt == PG_F32 ? 4 * L.r : dt == PG_BF16 ? 2 * L.r : L.r / 2;
}

// Table fields of a cache (any row count) for the layout.
int check_cache(const DevLayout& L, const pg_table* t, int32_t dt) {
  if (!t || !t->data || !aligned(t->data, 16) || t->dtype != dt || t->n_rows < 1)
    return PG_EINVAL;
  if (dt == PG_NF4 && (!t->scales || !aligned(t->scales, 2))) return PG_EINVAL;
  return PG_OK;
}

}  // namespace

PG_API int pg_stage_geometry(const pg_layout* layout, int32_t table_dtype, int32_t unit_kind,
                             int64_t n_tok, int64_t* unit_rows, int64_t* max_units,
                             int64_t* workspace_bytes) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  if (table_dtype != PG_F32 && table_dtype != PG_BF16 && table_dtype != PG_NF4) return PG_EINVAL;
  if (unit_kind != PG_STAGE_PAGE && unit_kind != PG_STAGE_ROW) return PG_EINVAL;
  if (n_tok < 0) return PG_EINVAL;
  if (n_tok > kMaxTokens) return PG_ERANGE;
  const int64_t U = stage_unit_rows(L, table_dtype, unit_kind);
  if (U > 65536) return PG_EUNSUPPORTED;
  const pg::StagePlan p = pg::stage_plan(L, (int)U, stage_share(L, unit_kind), n_tok);
  if (p.H > ((int64_t)1 << 31)) return PG_ERANGE;
  if (unit_rows) *unit_rows = U;
  if (max_units) *max_units = p.max_units;
  if (workspace_bytes) *workspace_bytes = p.bytes;
  return PG_OK;
}

PG_API int pg_stage_rows(const pg_layout* layout, const pg_table* src, int32_t unit_kind,
                         const int64_t* rows, int64_t n_tok, const pg_table* cache,
                         int64_t* cache_rows,
                         int64_t* n_units, int64_t* unit_first, void* workspace,
                         int64_t workspace_bytes, hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_table(L, src);
  if (st != PG_OK) return st;
  st = check_cache(L, cache, src->dtype);
  if (st != PG_OK) return st;
  int64_t U = 0, max_units = 0, ws_bytes = 0;
  st = pg_stage_geometry(layout, src->dtype, unit_kind, n_tok, &U, &max_units, &ws_bytes);
  if (st != PG_OK) return st;
  if (!n_units) return PG_EINVAL;
  if (n_tok == 0) return hip_status(pg::launch_set_i64(n_units, 0, stream));
  if (!rows || !cache_rows) return PG_EINVAL;
  if (cache->n_rows < max_units * U) return PG_EINVAL;
  if (!workspace || workspace_bytes < ws_bytes || !aligned(workspace, 256)) return PG_EINVAL;
  const pg::StagePlan p = pg::stage_plan(L, (int)U, stage_share(L, unit_kind), n_tok);
  return hip_status(pg::launch_stage(L, p, (int)data_row_bytes(L, src->dtype), src->data,
                                     src->scales, rows, const_cast<void*>(cache->data),
                                     const_cast<void*>(cache->scales), cache_rows, n_units,
                                     unit_first, workspace, stream));
}

PG_API int pg_gather_staged(const pg_layout* layout, const pg_table* cache,
                            const int64_t* cache_rows, const uint64_t* signs, int64_t n_tok,
                            int32_t e_dtype, void* e_out, hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  if (!cache) return PG_EINVAL;
  st = check_cache(L, cache, cache->dtype);
  if (st != PG_OK) return st;
  // the table's per-dtype row constraints, checked on a view with the
  // layout's row count
  pg_table view = *cache;
  view.n_rows = L.n_rows;
  st = check_table(L, &view);
  if (st != PG_OK) return st;
  if (e_dtype != table_e_dtype(cache->dtype)) return PG_EUNSUPPORTED;
  if (n_tok < 0) return PG_EINVAL;
  if (n_tok == 0) return PG_OK;
  if (!cache_rows || !signs || !e_out || !aligned(e_out, 16)) return PG_EINVAL;
  DevLayout LC = L;
  LC.n_rows = cache->n_rows;             // gather rows are clamped into the cache
  return hip_status(pg::launch_gather(LC, cache->dtype, cache->data, cache->scales, cache_rows,
                                      signs, n_tok, e_out, stream));
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) operands

PG_API int pg_quantize_fp8(const void* src, int32_t src_dtype, int64_t n, int32_t scale_exp,
                           uint8_t* dst, hipStream_t stream) {
  if (n < 0 || !scale_ok(scale_exp)) return PG_EINVAL;
  if (src_dtype != PG_BF16 && src_dtype != PG_F32) return PG_EINVAL;
  if (n == 0) return PG_OK;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return PG_EINVAL;
  return hip_status(pg::launch_quantize_fp8(src, src_dtype, n, scale_exp, dst, stream));
}

PG_API int pg_index_gather_fp8(const pg_layout* layout, const pg_table* table,
                               const int32_t* tokens, int64_t B, int64_t T,
                               const int32_t* canon_map, int64_t V, int32_t e_scale_exp,
                               uint8_t* e_out, int32_t* dev_status, hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_table(L, table);
  if (st != PG_OK) return st;
  st = check_tokens(tokens, B, T, canon_map, V);
  if (st != PG_OK) return st;
  if (!scale_ok(e_scale_exp)) return PG_EINVAL;
  if (B * T == 0) return PG_OK;
  if (!e_out || !aligned(e_out, 16)) return PG_EINVAL;
  return hip_status(pg::launch_index_gather(L, table->dtype, table->data, table->scales,
                                            tokens, B, T, canon_map, V, e_out, dev_status, 1,
                                            e_scale_exp, stream));
}

PG_API int pg_project_gate_fp8(const pg_fuse* fuse, const uint8_t* e8, int64_t B, int64_t T,
                               int64_t e_dim, const uint8_t* W8, int32_t e_scale_exp,
                               int32_t w_scale_exp, const void* resid, void* out,
                               void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  int st = check_fp8_fuse(fuse, B, T, e_dim, e_scale_exp, w_scale_exp);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!e8 || !W8 || !out) return PG_EINVAL;
  if (!aligned(e8, 16) || !aligned(W8, 16) || !aligned(out, 16)) return PG_EINVAL;
  if (resid && !aligned(resid, 16)) return PG_EINVAL;
  if (fuse->gate == PG_GATE_ENGRAM && !resid) return PG_EINVAL;
  const int64_t need = project_workspace(fuse, N);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return PG_EINVAL;
  return run_project_fp8(fuse, e8, B, T, e_dim, W8, e_scale_exp, w_scale_exp, resid, out,
                         workspace, stream);
}

PG_API int pg_forward_fp8(const pg_layout* layout, const pg_table* table, const pg_fuse* fuse,
                          const int32_t* tokens, int64_t B, int64_t T, const int32_t* canon_map,
                          int64_t V, const uint8_t* W8, int32_t e_scale_exp,
                          int32_t w_scale_exp, const void* resid, void* out, void* workspace,
                          int64_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
  DevLayout L;
  int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  st = check_table(L, table);
  if (st != PG_OK) return st;
  st = check_tokens(tokens, B, T, canon_map, V);
  if (st != PG_OK) return st;
  const int64_t e_dim = (int64_t)L.O * L.K * L.r;
  st = check_fp8_fuse(fuse, B, T, e_dim, e_scale_exp, w_scale_exp);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!W8 || !out || !aligned(W8, 16) || !aligned(out, 16)) return PG_EINVAL;
  if (resid && !aligned(resid, 16)) return PG_EINVAL;
  if (fuse->gate == PG_GATE_ENGRAM && !resid) return PG_EINVAL;
  const int64_t e_bytes = align256(N * e_dim);
  const int64_t need = e_bytes + project_workspace(fuse, N);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return PG_EINVAL;
  auto* e8 = static_cast<uint8_t*>(workspace);
  void* ws = e8 + e_bytes;
  st = hip_status(pg::launch_index_gather(L, table->dtype, table->data, table->scales, tokens,
                                          B, T, canon_map, V, e8, dev_status, 1, e_scale_exp,
                                          stream));
  if (st != PG_OK) return st;
  return run_project_fp8(fuse, e8, B, T, e_dim, W8, e_scale_exp, w_scale_exp, resid, out, ws,
                         stream);
}

// ---------------------------------------------------------------------------
// The Engram fusion's three stages (pg_project_gate runs them in order)

namespace {

// Checks shared by the stage calls: an Engram fuse, a workspace of
// pg_workspace_size(NULL, fuse, B, T) bytes.
int check_engram_stage(const pg_fuse* f, int64_t B, int64_t T, int64_t e_dim, const void* ws,
                       int64_t ws_bytes) {
  const int st = check_fuse(f, B, T, e_dim);
  if (st != PG_OK) return st;
  if (f->gate != PG_GATE_ENGRAM) return PG_EINVAL;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!ws || ws_bytes < project_workspace(f, N) || !aligned(ws, 256)) return PG_EINVAL;
  return PG_OK;
}

}  // namespace

PG_API int pg_engram_project(const pg_fuse* fuse, const void* e, int64_t B, int64_t T,
                             int64_t e_dim, const void* W, const void* h, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream) {
  const int st = check_engram_stage(fuse, B, T, e_dim, workspace, workspace_bytes);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!e || !W || !h || !aligned(e, 16) || !aligned(W, 16) || !aligned(h, 16)) return PG_EINVAL;
  return hip_status(pg::launch_engram_project(e, N, e_dim, W, fuse->d, fuse->M, fuse->gamma_h,
                                              fuse->gamma_k, h, workspace, 0, 0, 0, stream));
}

PG_API int pg_engram_project_fp8(const pg_fuse* fuse, const uint8_t* e8, int64_t B, int64_t T,
                                 int64_t e_dim, const uint8_t* W8, int32_t e_scale_exp,
                                 int32_t w_scale_exp, const void* h, void* workspace,
                                 int64_t workspace_bytes, hipStream_t stream) {
  int st = check_fp8_fuse(fuse, B, T, e_dim, e_scale_exp, w_scale_exp);
  if (st != PG_OK) return st;
  st = check_engram_stage(fuse, B, T, e_dim, workspace, workspace_bytes);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!e8 || !W8 || !h || !aligned(e8, 16) || !aligned(W8, 16) || !aligned(h, 16))
    return PG_EINVAL;
  return hip_status(pg::launch_engram_project(e8, N, e_dim, W8, fuse->d, fuse->M,
                                              fuse->gamma_h, fuse->gamma_k, h, workspace, 1,
                                              e_scale_exp, w_scale_exp, stream));
}

PG_API int pg_engram_gate(const pg_fuse* fuse, int64_t B, int64_t T, void* workspace,
                          int64_t workspace_bytes, hipStream_t stream) {
  // e_dim plays no part here; 64 passes the fuse check's e_dim rules
  const int st = check_engram_stage(fuse, B, T, 64, workspace, workspace_bytes);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  return hip_status(pg::launch_engram_gate(N, fuse->d, fuse->M, fuse->eps, workspace, stream));
}

PG_API int pg_engram_mix(const pg_fuse* fuse, int64_t B, int64_t T, const void* h, void* out,
                         void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  const int st = check_engram_stage(fuse, B, T, 64, workspace, workspace_bytes);
  if (st != PG_OK) return st;
  const int64_t N = B * T;
  if (N == 0) return PG_OK;
  if (!h || !out || !aligned(h, 16) || !aligned(out, 16)) return PG_EINVAL;
  return hip_status(pg::launch_engram_mix(B, T, fuse->d, fuse->M, fuse->gamma_u, fuse->conv_w,
                                          fuse->conv_k, fuse->conv_dil, h, out, workspace,
                                          fuse->increment_only ? 0 : 1, stream));
}

// ---------------------------------------------------------------------------
// Measurement

PG_API int pg_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes < 0 || bytes % 16) return PG_EINVAL;
  if (bytes == 0) return PG_OK;
  if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4)) return PG_EINVAL;
  return hip_status(pg::launch_read_probe(src, bytes, sink, kReadProbeBlocks, stream));
}

// ---------------------------------------------------------------------------
// Backward pass and table update

namespace {

// Shapes the backward pass supports; fills N, d, E, L.
int check_backward(const pg_layout* layout, const pg_fuse* fuse, int64_t B, int64_t T,
                   DevLayout* L, int64_t* N, int64_t* E, int64_t* Lk) {
  int st = prepare_layout(layout, L);
  if (st != PG_OK) return st;
  if (!fuse || B < 0 || T < 0) return PG_EINVAL;
  if (T > 0 && B > kMaxTokens / T) return PG_ERANGE;
  if (fuse->gate != PG_GATE_SCALAR || fuse->dtype != PG_BF16) return PG_EUNSUPPORTED;
  if (fuse->d < 64 || fuse->d % 64) return PG_EUNSUPPORTED;
  *N = B * T;
  *E = (int64_t)L->O * L->K * L->r;
  if (*E % 8) return PG_EUNSUPPORTED;
  *Lk = *N * L->O * L->K;
  if (*Lk >= ((int64_t)1 << 31) || L->n_rows > (int64_t)UINT32_MAX) return PG_ERANGE;
  return PG_OK;
}

}  // namespace

PG_API int64_t pg_backward_workspace_size(const pg_layout* layout, const pg_fuse* fuse,
                                          int64_t B, int64_t T) {
  DevLayout L;
  int64_t N, E, Lk;
  const int st = check_backward(layout, fuse, B, T, &L, &N, &E, &Lk);
  if (st != PG_OK) return st;
  return pg::backward_plan(N, fuse->d, E, Lk).bytes;
}

PG_API int pg_backward_scalar(const pg_layout* layout, const pg_fuse* fuse, const int64_t* rows,
                              const uint64_t* signs, const void* e, const void* dy,
                              const void* W, int64_t B, int64_t T, float* dW, float* de,
                              int64_t* urows, float* ugrad, int64_t* n_unique, void* workspace,
                              int64_t workspace_bytes, hipStream_t stream) {
  DevLayout L;
  int64_t N, E, Lk;
  int st = check_backward(layout, fuse, B, T, &L, &N, &E, &Lk);
  if (st != PG_OK) return st;
  if (!n_unique) return PG_EINVAL;
  if (N == 0) return hip_status(pg::launch_set_i64(n_unique, 0, stream));
  if (!rows || (L.use_signs && !signs) || !e || !dy || !W || !dW || !de || !urows || !ugrad)
    return PG_EINVAL;
  if (!aligned(e, 16) || !aligned(dy, 16) || !aligned(W, 16) || !aligned(dW, 16) ||
      !aligned(de, 16))
    return PG_EINVAL;
  const pg::BackwardPlan p = pg::backward_plan(N, fuse->d, E, Lk);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, 256)) return PG_EINVAL;
  return hip_status(pg::launch_backward_scalar(L, p, fuse->g, rows, signs, e, dy, W, N, fuse->d,
                                               dW, de, urows, ugrad, n_unique, workspace,
                                               stream));
}

PG_API int pg_row_rms_step(const pg_layout* layout, const int64_t* urows, const float* ugrad,
                           const int64_t* n_unique, int64_t max_unique, float* table, float* vhat,
                           int64_t* last_step, int64_t step, float lr, float beta2,
                           float weight_decay, float eps, hipStream_t stream) {
  DevLayout L;
  const int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  if (max_unique < 0 || step < 1 || !(lr >= 0.f) || !(beta2 >= 0.f && beta2 < 1.f) ||
      !(weight_decay >= 0.f) || !(eps >= 0.f) || lr * weight_decay >= 1.f)
    return PG_EINVAL;
  if (max_unique == 0) return PG_OK;
  if (!urows || !ugrad || !n_unique || !table || !vhat || !last_step) return PG_EINVAL;
  return hip_status(pg::launch_rms_step(urows, ugrad, n_unique, max_unique, L.r, table, vhat,
                                        last_step, step, lr, beta2, weight_decay, eps, stream));
}

PG_API int pg_row_rms_flush(const pg_layout* layout, float* table, float* vhat,
                            int64_t* last_step, int64_t step, float lr, float beta2,
                            float weight_decay, hipStream_t stream) {
  DevLayout L;
  const int st = prepare_layout(layout, &L);
  if (st != PG_OK) return st;
  if (step < 0 || !(lr >= 0.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(weight_decay >= 0.f) ||
      lr * weight_decay >= 1.f)
    return PG_EINVAL;
  if (L.n_rows == 0) return PG_OK;
  if (!table || !vhat || !last_step) return PG_EINVAL;
  return hip_status(pg::launch_rms_flush(L.n_rows, L.r, table, vhat, last_step, step, lr, beta2,
                                         weight_decay, stream));
}

}  // extern "C"
