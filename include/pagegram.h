/*
 * pagegram.h -- C ABI of the MI355X (gfx950) hashed multi-head n-gram memory
 * path: canonical IDs -> suffix n-grams -> multiply-XOR hashes -> PageGram or
 * Engram-style rows -> gather (fp32 / bf16 / NF4), +-1 signs, concatenation
 * -> W_V projection -> scalar-gated residual or Engram context gate with a
 * causal depthwise conv.
 *
 * Sources: PageGram tech report (Empero AI, 2026-10), sections 2.1-2.3, 3.1,
 * 3.3; Engram notes on "Conditional Memory via Scalable Lookup" (arXiv
 * 2601.07372), sections 3.2-3.4; Engram explainer (cooking-agi), lookup
 * pipeline and gate formulas.
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers are device memory owned by the
 *     caller, contiguous and row-major. The library allocates nothing and
 *     keeps no pointer after it returns. The only global state is
 *     pg_forward_noalloc's static device array and its per-GPU address,
 *     looked up once under a lock.
 *   - Work is enqueued on `stream` and the call returns without waiting;
 *     results are visible to later work on that stream.
 *   - Return value: PG_OK or a negative pg_status. Errors that the host can
 *     detect (NULL required pointers, bad sizes, misalignment, unsupported
 *     shapes) are returned before anything is enqueued. PG_EHIP means a HIP
 *     launch failed.
 *   - Token IDs outside [0, V) are treated as the layout's pad_id and set
 *     bit 0 of *dev_status (an int32 in device memory, OR-ed with
 *     atomicOr; never cleared by the library) when dev_status is non-NULL.
 *     Every row is reduced modulo its sub-table size, so no input value can
 *     make the gather read outside the table.
 *   - N = B*T tokens; B rows of T tokens are separate sequences (no n-gram
 *     and no convolution crosses a row). N = 0 is valid and enqueues nothing.
 */
#ifndef PAGEGRAM_H
#define PAGEGRAM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PG_API __attribute__((visibility("default")))
#else
#define PG_API
#endif

typedef enum pg_status {
  PG_OK = 0,
  PG_EINVAL = -1,        /* NULL required pointer, bad size or alignment   */
  PG_EUNSUPPORTED = -2,  /* valid but not implemented (shape, dtype combo) */
  PG_EHIP = -3,          /* a HIP call or kernel launch failed             */
  PG_ERANGE = -4         /* a size overflows the library's index types     */
} pg_status;

typedef enum pg_layout_kind {
  PG_PAGEGRAM = 0,  /* page-local heads: PageGram §3.1                      */
  PG_ENGRAM = 1     /* one sub-table per head: PageGram §2.2, Engram §3.2    */
} pg_layout_kind;

typedef enum pg_dtype { PG_F32 = 0, PG_BF16 = 1, PG_NF4 = 2 } pg_dtype;

typedef enum pg_gate {
  PG_GATE_SCALAR = 0,  /* x <- x + g * W_V e             (PageGram §3.1)   */
  PG_GATE_ENGRAM = 1   /* context gate + conv, M branches (Engram §3.3-3.4) */
} pg_gate;

#define PG_MAX_ORDERS 4
#define PG_MAX_HEADS 16

/*
 * Layout of the n-gram table T in R^{R x r} and its hash functions.
 *
 * Orders n = n_min..n_max (1 <= n_min <= n_max <= 4); O = n_max-n_min+1.
 * PageGram (PageGram §3.1): order n owns pages[n-n_min] = P_n pages of K*S
 *   rows; base_n are cumulative in order of n;
 *     p_n = b_n(x) mod P_n,
 *     row_{n,k} = base_n + (p_n*K + k)*S + (u_{n,k}(x) mod S).
 * Engram-style (PageGram §2.2): head (n,k) owns head_rows[n-n_min][k] =
 *   P_{n,k} rows; bases cumulative in (n, k) order;
 *     row_{n,k} = base_{n,k} + (u_{n,k}(x) mod P_{n,k}).
 * The flat table of PageGram §2.1 is PG_PAGEGRAM with K=1, S=1.
 *
 * Hashes (hash version 1; the Engram notes, section 3.2, fix only a light
 * multiply-XOR hash per head, and the PageGram tech report, section 3.1, a
 * page hash b_n beside the head hashes u_{n,k}): for an n-gram
 * g_j = canonical ID at position t-j (j = 0..n-1; pad_id before the start of
 * the sequence) and a role (page hash b_n, head hash u_{n,k}, sign word w of
 * head (n,k)):
 *     h = mix64(c XOR (a_0*g_0) XOR ... XOR (a_{n-1}*g_{n-1}))   (mod 2^64)
 * where mix64 is splitmix64's output function and, with
 * idx = ((n*4 + kind)*64 + k)*8 + w (kind 0 page, 1 head, 2 sign),
 *     c   = splitmix64 output 8*idx       of the stream seeded by hash_seed,
 *     a_j = splitmix64 output 8*idx+1+j   with its low bit set.
 * Signs (PageGram §2.1, §3.1): element j of head (n,k) is -1 when bit j%64
 * of sign word j/64 is set, +1 otherwise; use_signs = 0 makes all signs +1.
 *
 * Limits: 1 <= K <= 16; S >= 1; r >= 1 with r <= 256; every P >= 1 and the
 * total row count R < 2^62.
 */
typedef struct pg_layout {
  int32_t kind;                 /* pg_layout_kind                          */
  int32_t n_min, n_max;         /* n-gram orders                           */
  int32_t K;                    /* heads per order                         */
  int32_t S;                    /* slots per head per page (PageGram)      */
  int32_t r;                    /* head row width in elements              */
  int64_t pages[PG_MAX_ORDERS]; /* P_n (PageGram)                          */
  int64_t head_rows[PG_MAX_ORDERS][PG_MAX_HEADS]; /* P_{n,k} (Engram-style) */
  uint64_t hash_seed;
  int32_t use_signs;            /* 1: hash-derived +-1 signs; 0: none      */
  int32_t pad_id;               /* canonical ID before a sequence start;
                                   normally the canonical vocabulary size V' */
} pg_layout;

/*
 * Table storage (device memory, 16-byte aligned).
 *   PG_F32 / PG_BF16: data = [n_rows][r] elements; r*elt must be a multiple
 *     of 16 bytes.
 *   PG_NF4 (PageGram §2.3, §3.3: 64 4-bit codes + one fp16 scale = 34 B per
 *     64-wide row): data = [n_rows][r/2] bytes of codes, code j of a row in
 *     byte j/2, low nibble for even j; scales = fp16 [n_rows]; r a multiple
 *     of 32. Value = nf4[code] * scale with QLoRA's NormalFloat levels; a
 *     page's codes (K*S*r/2 bytes) and its scales (K*S*2 bytes) are each
 *     contiguous.
 * n_rows must equal pg_layout_rows().
 */
typedef struct pg_table {
  int32_t dtype;                /* pg_dtype                                */
  int32_t reserved;             /* 0                                       */
  const void* data;
  const void* scales;           /* NF4 only, else NULL                     */
  int64_t n_rows;
} pg_table;

/*
 * Projection and fusion stage.
 *   dtype: element type of e, W, the residual and the output: PG_F32 (with
 *     an fp32 table) or PG_BF16 (bf16 or NF4 table). Accumulation is fp32.
 *   Scalar gate (PageGram §3.1): out = resid + g * (W e), W = W_V [d x E].
 *   Engram gate (Engram §3.3-3.4, M branches; W = [W_V; W_K^(1..M)] with
 *   (1+M)*d rows; resid = h [M][N][d]; out [M][N][d]):
 *     v = W_V e, k^m = W_K^(m) e,
 *     alpha^m = sigmoid(RMSNorm_h(h^m) . RMSNorm_k(k^m) / sqrt(d)),
 *     u^m = alpha^m v,
 *     out^m = h^m + u^m + SiLU(CausalDWConv(RMSNorm_u(u^m))),
 *   RMSNorm_x(z) = gamma_x * z / sqrt(mean(z^2) + eps), gains shared by the
 *   branches; conv per channel c:
 *     y_t[c] = sum_{j<conv_k} conv_w[c][j] * z_{t-(conv_k-1-j)*conv_dil}[c],
 *   zero before the start of the sequence. gamma_* = fp32 [d] and conv_w =
 *   fp32 [d][conv_k], device memory. Engram needs dtype PG_BF16, d a
 *   multiple of 256, e_dim a multiple of 64, 1 <= M <= 8, 1 <= conv_k <= 8
 *   and (conv_k-1)*conv_dil <= 64.
 *   increment_only = 1 writes the increment alone (g*W e, or
 *   u^m + SiLU(...)) without adding the residual; the Engram gate still
 *   reads h for alpha. For the scalar gate a NULL resid acts as zero.
 */
typedef struct pg_fuse {
  int32_t gate;                 /* pg_gate                                 */
  int32_t dtype;                /* PG_F32 or PG_BF16                       */
  int32_t d;                    /* model width (output columns per branch) */
  int32_t M;                    /* Engram branches (ignored for scalar)    */
  float g;                      /* scalar gate                             */
  float eps;                    /* RMSNorm epsilon                         */
  const float* gamma_h;
  const float* gamma_k;
  const float* gamma_u;
  const float* conv_w;
  int32_t conv_k;
  int32_t conv_dil;
  int32_t increment_only;       /* 0: out = resid + increment; 1: increment */
  int32_t reserved;             /* 0                                       */
} pg_fuse;

/*
 * pg_index -- addresses only (canonical map, n-grams, hashes, rows, signs).
 * Touches no table, so it can run ahead of the forward (PageGram §3.3,
 * prefetch; Engram §3.5).
 *   tokens     int32 [B][T] (device)
 *   canon_map  int32 [V]    (device), values < 2^31
 *   canon_out  int32 [N]            nullable
 *   hash_out   uint64 [N][O][1+K]   nullable: (b_n, u_{n,0..K-1})
 *   rows_out   int64 [N][O][K]      required
 *   pages_out  int64 [N][O]         nullable: p_n, or -1 (Engram-style)
 *   signs_out  uint64 [N][O][K][ceil(r/64)]  required (zeros if no signs)
 *   dev_status int32 [1]            nullable
 */
PG_API int pg_index(const pg_layout* layout, const int32_t* tokens, int64_t B,
                    int64_t T, const int32_t* canon_map, int64_t V,
                    int32_t* canon_out, uint64_t* hash_out, int64_t* rows_out,
                    int64_t* pages_out, uint64_t* signs_out,
                    int32_t* dev_status, hipStream_t stream);

/*
 * pg_gather -- e[t] = concat_{n, then k} s_{n,k} * deq(T[row_{n,k}(t)])
 * (PageGram §2.2, §3.1; Engram §3.2) from pg_index's rows and signs.
 *   rows   int64 [n_tok][O][K] (device), each in [0, n_rows)
 *   signs  uint64 [n_tok][O][K][ceil(r/64)] (device); may be NULL only when
 *          use_signs = 0
 *   e_dtype PG_F32 for an fp32 table, PG_BF16 for bf16 and NF4 tables
 *   e_out  [n_tok][O*K*r] (device, 16-byte aligned)
 * NF4 values are fp32(nf4[code]*scale) rounded to bf16 (nearest even).
 * Rows outside [0, n_rows) are clamped to the last row (never read out of
 * bounds) -- pg_index never produces them.
 */
PG_API int pg_gather(const pg_layout* layout, const pg_table* table,
                     const int64_t* rows, const uint64_t* signs, int64_t n_tok,
                     int32_t e_dtype, void* e_out, hipStream_t stream);

/*
 * pg_index_gather -- pg_index followed by pg_gather in one kernel, with the
 * rows and signs kept on chip: tokens -> e. Same arguments and results as
 * the pair.
 */
PG_API int pg_index_gather(const pg_layout* layout, const pg_table* table,
                           const int32_t* tokens, int64_t B, int64_t T,
                           const int32_t* canon_map, int64_t V,
                           int32_t e_dtype, void* e_out, int32_t* dev_status,
                           hipStream_t stream);

/*
 * pg_project_gate -- projection through W and the fusion stage: the
 * scalar-gated residual of the PageGram tech report (section 3.1: the memory
 * vector is projected by W_V and added to the residual stream through a
 * learned scalar gate), or the Engram notes' context gate, convolution and
 * branch integration (sections 3.3-3.4), as defined under pg_fuse above.
 *   e        [N][e_dim]              (device, fuse->dtype)
 *   W        [d_out][e_dim]          (device, fuse->dtype), d_out = d, or
 *                                    (1+M)*d for the Engram gate
 *   resid    x [N][d] (nullable), or h [M][N][d] (required for the
 *            Engram gate)            (device, fuse->dtype)
 *   out      [N][d], or [M][N][d]    (device, fuse->dtype)
 *   workspace at least pg_workspace_size(NULL, fuse, B, T) bytes of device
 *            memory (256-byte aligned); may be NULL when that size is 0
 * e_dim must be a multiple of 8 (bf16) or 4 (fp32); all pointers 16-byte
 * aligned.
 */
PG_API int pg_project_gate(const pg_fuse* fuse, const void* e, int64_t B,
                           int64_t T, int64_t e_dim, const void* W,
                           const void* resid, void* out, void* workspace,
                           int64_t workspace_bytes, hipStream_t stream);

/*
 * pg_index_records -- the addressing half of the gathered projection
 * (PageGram §3.1 rows and the Engram notes' per-head rows; the signs of
 * §3.1): for every head slot hs = (n - n_min) K + k and token t, a
 * 16-byte record at rec_out + (hs B T + t) 16 holding the row and the
 * head's sign bits in the order pg_project_gathered's matrix-core fragments
 * consume them (a format private to the library). Rows of 64 elements only
 * (PG_EUNSUPPORTED otherwise); B T at most 2^28 (PG_ERANGE). rec_out is
 * B T n_ord K 16 bytes of device memory, 16-byte aligned. Tokens outside
 * [0, V) as for pg_index.
 */
PG_API int pg_index_records(const pg_layout* layout, const int32_t* tokens,
                            int64_t B, int64_t T, const int32_t* canon_map,
                            int64_t V, void* rec_out, int32_t* dev_status,
                            hipStream_t stream);

/*
 * pg_project_gathered -- the scalar-gate projection (PageGram §3.1:
 * out = x + g W e) with e gathered from the table inside the matrix
 * kernel by pg_index_records' records, so e never goes to memory. Same
 * results, bit for bit, as pg_gather followed by pg_project_gate. bf16
 * tables of 64-element rows with at most 2^25 rows, fuse->dtype bf16 and
 * the scalar gate (PG_EUNSUPPORTED otherwise). W, resid (nullable) and out
 * as for pg_project_gate; all pointers 16-byte aligned.
 */
PG_API int pg_project_gathered(const pg_layout* layout, const pg_table* table,
                               const pg_fuse* fuse, const void* rec, int64_t B,
                               int64_t T, const void* W, const void* resid,
                               void* out, hipStream_t stream);

/*
 * pg_forward -- the whole path, tokens -> out: the lookup pipeline of the
 * Engram explainer (canonical IDs, suffix n-grams, several hashes, table
 * rows, concatenated e_t), addressed as in the PageGram tech report section
 * 3.1 or the Engram notes section 3.2, then the fusion of pg_project_gate.
 * Equal to pg_index_gather
 * followed by pg_project_gate up to float summation order (bit for bit
 * where it runs as pg_index_records followed by pg_project_gathered: bf16
 * tables of 64-element rows under the scalar gate). workspace at least
 * pg_workspace_size(layout, fuse, B, T) bytes (256-byte aligned).
 */
PG_API int pg_forward(const pg_layout* layout, const pg_table* table,
                      const pg_fuse* fuse, const int32_t* tokens, int64_t B,
                      int64_t T, const int32_t* canon_map, int64_t V,
                      const void* W, const void* resid, void* out,
                      void* workspace, int64_t workspace_bytes,
                      int32_t* dev_status, hipStream_t stream);

/*
 * pg_forward_noalloc -- pg_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same results, bit for bit, with
 * the workspace taken from a static device array of PG_NOALLOC_SCRATCH_BYTES
 * that the library's code object holds on every GPU it runs on until the
 * process ends. No allocating call is made. The arguments are pg_forward's
 * without workspace and workspace_bytes. PG_ERANGE when
 * pg_workspace_size(layout, fuse, B, T) exceeds PG_NOALLOC_SCRATCH_BYTES
 * (the 200M-parameter workloads' 8 x 2048 tokens fit; the 20B and 27B ones do
 * not). All calls on one GPU share the array: calls that overlap on one GPU
 * (other streams, other host threads) race and must be ordered by the caller.
 * The array's device address is looked up on the first call on a GPU (with
 * that GPU made current for the lookup); PG_EHIP if the lookup fails.
 */
#define PG_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)

PG_API int pg_forward_noalloc(const pg_layout* layout, const pg_table* table,
                              const pg_fuse* fuse, const int32_t* tokens,
                              int64_t B, int64_t T, const int32_t* canon_map,
                              int64_t V, const void* W, const void* resid,
                              void* out, int32_t* dev_status,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * The Engram gate's three stages (Engram notes §3.3-3.4: the value and key
 * projections of e, the context gate alpha^m per branch, then the causal
 * depthwise conv, SiLU and residual; Engram explainer, gate formulas).
 * pg_project_gate with the Engram gate is exactly pg_engram_project,
 * pg_engram_gate and pg_engram_mix in that order, on one workspace of
 * pg_workspace_size(NULL, fuse, B, T) bytes (256-byte aligned) that carries
 * the intermediate values between them: v = W_V e in bf16 and per-token
 * partial sums (sum v^2; per branch sum k^2, sum gamma_h gamma_k h k,
 * sum h^2 over 256-column blocks), then alpha^m and the RMSNorm_u scale.
 * The workspace's contents between the calls are private to the library.
 * fuse->gate must be PG_GATE_ENGRAM (PG_EINVAL otherwise) with the limits
 * of pg_fuse; N = 0 enqueues nothing.
 * ------------------------------------------------------------------------ */

/*
 * pg_engram_project -- the fused projection [W_V; W_K^(1..M)] e (pass 1):
 * v and the partial sums into the workspace; k^m is reduced on chip and
 * never stored.
 *   e  [N][e_dim] bf16, W [(1+M) d][e_dim] bf16, h [M][N][d] bf16 (device,
 *   16-byte aligned).
 */
PG_API int pg_engram_project(const pg_fuse* fuse, const void* e, int64_t B,
                             int64_t T, int64_t e_dim, const void* W,
                             const void* h, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream);

/*
 * pg_engram_project_fp8 -- pg_engram_project on E4M3 operands e8 and W8
 * (scales as for pg_project_gate_fp8; e_dim a multiple of 128).
 */
PG_API int pg_engram_project_fp8(const pg_fuse* fuse, const uint8_t* e8,
                                 int64_t B, int64_t T, int64_t e_dim,
                                 const uint8_t* W8, int32_t e_scale_exp,
                                 int32_t w_scale_exp, const void* h,
                                 void* workspace, int64_t workspace_bytes,
                                 hipStream_t stream);

/*
 * pg_engram_gate -- per (branch, token): alpha^m = sigmoid(RMSNorm_h(h^m) .
 * RMSNorm_k(k^m) / sqrt(d)) and alpha^m / sqrt(alpha^m^2 mean(v^2) + eps)
 * from the partial sums pg_engram_project left in the workspace.
 */
PG_API int pg_engram_gate(const pg_fuse* fuse, int64_t B, int64_t T,
                          void* workspace, int64_t workspace_bytes,
                          hipStream_t stream);

/*
 * pg_engram_mix -- pass 2: out^m = h^m + u^m + SiLU(CausalDWConv(
 * RMSNorm_u(u^m))) with u^m = alpha^m v (increment_only drops h^m), from
 * the workspace pg_engram_gate completed.
 *   h, out [M][N][d] bf16 (device, 16-byte aligned).
 */
PG_API int pg_engram_mix(const pg_fuse* fuse, int64_t B, int64_t T,
                         const void* h, void* out, void* workspace,
                         int64_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Staging from a host-resident table (PageGram tech report §3.3, Engram
 * notes §3.5: addresses depend only on token IDs and are known before the
 * layer runs, so the touched parts of a table kept in host memory can be
 * fetched ahead). The unit of transfer is a PageGram page (K*S rows, shared
 * by the K heads of a token-order) or, for the Engram-style tables, a run of
 * floor(4096 / row_bytes) rows of one per-head table starting at that
 * table's first row (row_bytes: fp32 4r, bf16 2r, NF4 r/2 + 2).
 * ------------------------------------------------------------------------ */

/* Unit of transfer: the page / 4 KiB run above, or single rows. */
enum pg_stage_unit { PG_STAGE_PAGE = 0, PG_STAGE_ROW = 1 };

/*
 * pg_stage_geometry -- rows per unit U, the most units a step of n_tok tokens
 * can touch (n_tok * orders for PageGram pages, n_tok * orders * K
 * otherwise), and the device workspace bytes of pg_stage_rows. Outputs are
 * host pointers, each nullable.
 */
PG_API int pg_stage_geometry(const pg_layout* layout, int32_t table_dtype, int32_t unit_kind,
                             int64_t n_tok, int64_t* unit_rows, int64_t* max_units,
                             int64_t* workspace_bytes);

/*
 * pg_stage_rows -- copy every unit (of kind unit_kind) that rows touch, once,
 * from src into a device cache, and rewrite the rows for it.
 *   src         the whole table (pg_table as above); data (and NF4 scales)
 *               must be readable by the device: device memory, or pinned
 *               host memory allocated with hipHostMalloc
 *   rows        [n_tok][orders][K] int64 device (pg_index's rows_out)
 *   cache       device table of src's dtype with n_rows >= max_units * U;
 *               unit s of the step occupies rows [s U, s U + its rows)
 *   cache_rows  [n_tok][orders][K] int64 device: the row of each lookup in
 *               the cache (cache row cache_rows[q] holds table row rows[q])
 *   n_units     int64 device: the number of units staged
 *   unit_first  int64 device [max_units], nullable: first table row of the
 *               unit in each slot (slots follow a deterministic order)
 *   workspace   pg_stage_geometry bytes of device memory, 256-byte aligned
 * Rows outside [0, R) are clamped into the table.
 */
PG_API int pg_stage_rows(const pg_layout* layout, const pg_table* src, int32_t unit_kind,
                         const int64_t* rows, int64_t n_tok, const pg_table* cache,
                         int64_t* cache_rows,
                         int64_t* n_units, int64_t* unit_first, void* workspace,
                         int64_t workspace_bytes, hipStream_t stream);

/*
 * pg_gather_staged -- pg_gather from a cache filled by pg_stage_rows: e from
 * (cache, cache_rows, signs) equals pg_gather's e from (table, rows, signs)
 * bit for bit. cache->n_rows is the cache's own row count.
 */
PG_API int pg_gather_staged(const pg_layout* layout, const pg_table* cache,
                            const int64_t* cache_rows, const uint64_t* signs, int64_t n_tok,
                            int32_t e_dtype, void* e_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 operands (Engram notes §3.4: the value and key projections run as one
 * dense FP8 GEMM). Format: OCP E4M3 (sign, 4-bit exponent of bias 7, 3-bit
 * mantissa, no infinities, 0x7F / 0xFF NaN, largest finite 448). A tensor
 * is stored as q = E4M3(v * 2^s) with one power-of-two scale exponent s per
 * tensor chosen by the caller (|s| <= 64): rounded to nearest, ties to the
 * even mantissa; magnitudes at or above 448 saturate to 448; NaN stays NaN;
 * the sign of zero is kept. The projection multiplies the dequantised
 * operands q 2^-s on the matrix cores with fp32 accumulation; residual and
 * output stay bf16.
 * ------------------------------------------------------------------------ */

/*
 * pg_quantize_fp8 -- dst[i] = E4M3(src[i] * 2^scale_exp), i < n (W, say).
 *   src  [n] device, PG_BF16 or PG_F32 (src_dtype), 16-byte aligned
 *   dst  [n] device bytes, 16-byte aligned
 */
PG_API int pg_quantize_fp8(const void* src, int32_t src_dtype, int64_t n,
                           int32_t scale_exp, uint8_t* dst, hipStream_t stream);

/*
 * pg_index_gather_fp8 -- pg_index_gather writing e as E4M3 bytes:
 * e_out[t][j] = E4M3(e[t][j] * 2^e_scale_exp), where e is the value
 * pg_index_gather stores (bf16 for bf16 and NF4 tables -- NF4 rounded to
 * bf16 first -- fp32 for an fp32 table). e_out [B*T][e_dim] device bytes,
 * 16-byte aligned.
 */
PG_API int pg_index_gather_fp8(const pg_layout* layout, const pg_table* table,
                               const int32_t* tokens, int64_t B, int64_t T,
                               const int32_t* canon_map, int64_t V,
                               int32_t e_scale_exp, uint8_t* e_out,
                               int32_t* dev_status, hipStream_t stream);

/*
 * pg_project_gate_fp8 -- pg_project_gate on E4M3 operands:
 *   e8  [N][e_dim] = E4M3(e 2^e_scale_exp), W8 [d_out][e_dim] =
 *   E4M3(W 2^w_scale_exp) (device bytes); resid / out bf16 as in
 *   pg_project_gate (fuse->dtype must be PG_BF16); e_dim a multiple of 128;
 *   workspace as for pg_project_gate. PG_EUNSUPPORTED otherwise.
 */
PG_API int pg_project_gate_fp8(const pg_fuse* fuse, const uint8_t* e8, int64_t B,
                               int64_t T, int64_t e_dim, const uint8_t* W8,
                               int32_t e_scale_exp, int32_t w_scale_exp,
                               const void* resid, void* out, void* workspace,
                               int64_t workspace_bytes, hipStream_t stream);

/*
 * pg_forward_fp8 -- pg_index_gather_fp8 followed by pg_project_gate_fp8;
 * workspace at least pg_workspace_size(layout, fuse, B, T) bytes (256-byte
 * aligned; e takes one byte per element here).
 */
PG_API int pg_forward_fp8(const pg_layout* layout, const pg_table* table,
                          const pg_fuse* fuse, const int32_t* tokens, int64_t B,
                          int64_t T, const int32_t* canon_map, int64_t V,
                          const uint8_t* W8, int32_t e_scale_exp,
                          int32_t w_scale_exp, const void* resid, void* out,
                          void* workspace, int64_t workspace_bytes,
                          int32_t* dev_status, hipStream_t stream);

/*
 * pg_read_probe -- measurement utility, not part of the path: reads `bytes`
 * (a multiple of 16) at src once with 16-byte streaming loads, 4,096 blocks
 * each reading one contiguous chunk, and writes the XOR of the 32-bit words
 * each block read into sink (device, 4,096 uint32; the XOR of all sink words
 * is the XOR of all words of the buffer). Timed by the caller, it gives the
 * read rate the GPU sustains, the measured ceiling quoted beside the HBM
 * specification.
 */
PG_API int pg_read_probe(const void* src, int64_t bytes, uint32_t* sink,
                         hipStream_t stream);

/* Message for a pg_status value (static storage). */
PG_API const char* pg_strerror(int status);

/*
 * Hash definition version implemented (1, as described under pg_layout).
 * The pages fix the hash only as a light multiply-XOR per head (Engram
 * notes section 3.2; the PageGram tech report section 3.1 adds a separate
 * page hash b_n next to the head hashes u_{n,k}); the constants and the
 * splitmix64 finaliser are this library's choice, so the version names the
 * bit-level definition a stored table was trained with.
 */
PG_API uint32_t pg_hash_version(void);

/* Total row count R of a layout; PG_EINVAL / PG_ERANGE for a bad layout. */
PG_API int pg_layout_rows(const pg_layout* layout, int64_t* n_rows);

/*
 * Workspace bytes needed by pg_forward (layout non-NULL) or by
 * pg_project_gate (layout NULL) for B x T tokens; negative pg_status on bad
 * arguments.
 */
PG_API int64_t pg_workspace_size(const pg_layout* layout, const pg_fuse* fuse,
                                 int64_t B, int64_t T);

/* ------------------------------------------------------------------------
 * Backward pass of the scalar-gated path and the sparse table update
 * (PageGram tech report §3.3: tables start at zero, a row-wise adaptive RMS
 * optimiser with replayed decay; §9.1: beta2 = 0.95; §9.4 check 4: the
 * sparse gradient equals the dense one). Readings where the pages are
 * silent: v is one scalar per row (moving average of the row's mean squared
 * gradient), no bias correction, a step divides by sqrt(v) + eps and applies
 * decoupled weight decay.
 * ------------------------------------------------------------------------ */

/*
 * pg_backward_workspace_size -- device workspace bytes of pg_backward_scalar
 * for B x T tokens (negative pg_status for unsupported shapes: the scalar
 * gate, bf16 activations, d a multiple of 64, e_dim a multiple of 8, fewer
 * than 2^31 lookups and 2^32 rows).
 */
PG_API int64_t pg_backward_workspace_size(const pg_layout* layout, const pg_fuse* fuse,
                                          int64_t B, int64_t T);

/*
 * pg_backward_scalar -- gradients of out = x + g W e (fuse->g) given
 * dy = dL/dout:
 *   de  fp32 [B*T][e_dim] = g dy W
 *   dW  fp32 [d][e_dim]   = g dy^T e  (summed over tokens in a fixed order)
 *   table gradient restricted to the touched rows: urows int64 [*n_unique]
 *   ascending, ugrad fp32 [*n_unique][r]; ugrad[u] is the sum over the
 *   lookups (t, n, k) with rows[t][n][k] = urows[u], in lookup order, of
 *   s_{t,n,k} (.) de[t][(n,k) slice].
 *   rows, signs: pg_index's outputs for these tokens; e: the forward's e
 *   (bf16 [B*T][e_dim]); dy bf16 [B*T][d]; W bf16 [d][e_dim] (device).
 *   urows / ugrad need room for B*T*O*K entries; n_unique is a device int64.
 * Deterministic (no floating-point atomics). Errors: PG_EUNSUPPORTED for the
 * shapes pg_backward_workspace_size rejects, PG_EINVAL for NULL or
 * misaligned (16 B) pointers or a short workspace (256-byte aligned).
 */
PG_API int pg_backward_scalar(const pg_layout* layout, const pg_fuse* fuse,
                              const int64_t* rows, const uint64_t* signs, const void* e,
                              const void* dy, const void* W, int64_t B, int64_t T,
                              float* dW, float* de, int64_t* urows, float* ugrad,
                              int64_t* n_unique, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream);

/*
 * pg_row_rms_step -- one optimiser step at step number `step` (>= 1) on the
 * rows urows[0 .. *n_unique) with gradients ugrad (pg_backward_scalar's
 * outputs; max_unique bounds *n_unique). For a row last updated at step
 * tau (last_step[row], 0 when never), with k = step - tau:
 *   v     <- beta2^k v + (1 - beta2) mean_j(g_j^2)
 *   theta <- theta (1 - lr wd)^k - lr g / (sqrt(v) + eps)
 *   last_step[row] <- step
 * (the k - 1 skipped steps replayed as decay, then this step).
 *   table fp32 [R][r] (the master copy of the table), vhat fp32 [R],
 *   last_step int64 [R] (device; zero-initialised by the caller).
 * Errors: PG_EINVAL for bad hyper-parameters (beta2 outside [0, 1),
 * lr * wd >= 1, negative values) or NULL pointers.
 */
PG_API int pg_row_rms_step(const pg_layout* layout, const int64_t* urows,
                           const float* ugrad, const int64_t* n_unique, int64_t max_unique,
                           float* table, float* vhat, int64_t* last_step, int64_t step,
                           float lr, float beta2, float weight_decay, float eps,
                           hipStream_t stream);

/*
 * pg_row_rms_flush -- brings every row to `step`: theta *= (1 - lr wd)^k,
 * v *= beta2^k, last_step = step, with k = step - last_step[row] (rows
 * already at step untouched). After it the table equals the one a dense
 * optimiser (every row every step, zero gradients for untouched rows)
 * would hold.
 */
PG_API int pg_row_rms_flush(const pg_layout* layout, float* table, float* vhat,
                            int64_t* last_step, int64_t step, float lr, float beta2,
                            float weight_decay, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Flash page-cache simulation (host code; PageGram tech report §2.3, §3.3,
 * §8 Fig. 4a and appendix D). A table kept on flash is read in 4 KiB blocks;
 * a RAM page cache with LRU replacement holds whole blocks; each lookup whose
 * block is not cached is one random flash read.
 * ------------------------------------------------------------------------ */

/*
 * pg_flash_blocks -- the 4 KiB block holding each looked-up row, in the
 * pages' storage order. PageGram: a page is K*S consecutive head rows; when a
 * page fits in a block, floor(4096 / page_bytes) whole pages share a block
 * (three 1,088-byte NF4 pages at S = 4, one 4,080-byte page at S = 15),
 * otherwise a page spans ceil(page_bytes / 4096) blocks and a row lies in
 * the block of its byte offset. Engram-style: each per-head table starts on
 * a fresh block and packs floor(4096 / row_bytes) rows per block (120 NF4
 * rows of 34 bytes).
 *   table_dtype  PG_F32 / PG_BF16 / PG_NF4 (row bytes 4r / 2r / r/2 + 2)
 *   rows         host int64 [n] row indices (e.g. pg_index's rows, copied
 *                to the host); blocks_out host int64 [n].
 * Errors: PG_EINVAL for a bad layout, dtype or NULL pointer with n > 0;
 * PG_ERANGE for a row outside [0, R). Thread-safe, allocates nothing.
 */
PG_API int pg_flash_blocks(const pg_layout* layout, int32_t table_dtype,
                           const int64_t* rows, int64_t n, int64_t* blocks_out);

/* Counters of one LRU run. */
typedef struct {
  int64_t tokens;     /* tokens offered */
  int64_t lookups;    /* row lookups (tokens * per_token) */
  int64_t distinct;   /* sum over tokens of distinct blocks (uncached reads) */
  int64_t misses;     /* flash reads with the cache */
} pg_cache_stats;

/*
 * pg_lru_cache_sim -- offers each token's distinct blocks (first-use order,
 * duplicates within the token dropped) to an LRU cache of capacity_blocks
 * 4 KiB blocks (0 = no cache) and counts the misses.
 *   blocks  host int64 [n_tok][per_token] (pg_flash_blocks of [n_tok][O][K]
 *           rows; per_token = O * K)
 * Errors: PG_EINVAL for NULL pointers with n_tok > 0, per_token < 1 or a
 * negative capacity. Allocates host memory for the cache state only for the
 * duration of the call; thread-safe.
 */
PG_API int pg_lru_cache_sim(const int64_t* blocks, int64_t n_tok, int32_t per_token,
                            int64_t capacity_blocks, pg_cache_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* PAGEGRAM_H */
