"""CPU oracle of the hashed multi-head n-gram memory hot path.

TEST INFRASTRUCTURE ONLY. This module is imported by the tests, by the smoke
check and by the benchmark's CPU-baseline leg, and by nothing on the product
path. It shares no code with the HIP library: it re-derives every constant
itself and takes its inputs (token IDs, canonical map, table rows, weights,
residual inputs) from the caller.

Plain and slow on purpose: numpy, exact unsigned 64-bit integers for
canonical IDs, hashes, rows and pages, float64 for all floating point. Each
step follows the pages in their order:

  canonical map -> suffix n-grams -> multiply-XOR hashes -> rows (PageGram or
  Engram-style) -> gather, dequantise, sign, concatenate -> W_V projection ->
  scalar-gated residual, or the Engram context gate + RMSNorm + causal
  depthwise conv + SiLU + skip.

Sources: the PageGram tech report (Empero AI, 2026-10) sections 2.1-2.3, 3.1,
3.3, 4; the Engram explainer (cooking-agi, "Engram") lookup pipeline and gate
formulas; the Engram notes on "Conditional Memory via Scalable Lookup"
(arXiv 2601.07372) sections 3.2-3.4.

Where the pages leave a step open the readings taken are:
  * hash family: multiply-XOR with a splitmix64 output function as finaliser,
    constants drawn from a splitmix64 stream of the hash seed (role_constants);
  * positions before a sequence's start hash as the PAD id (= canonical
    vocabulary size); no n-gram crosses a batch row;
  * sign bits: element j of a head uses bit j%64 of sign word j//64,
    bit 1 -> -1;
  * NF4 codebook: QLoRA's asymmetric normal-quantile construction; parity with
    QLoRA's own printed table is unpinned (it is not on the pages);
  * Engram gains are shared by the M branches, conv follows torch conv1d
    (cross-correlation, left zero padding, groups = channels).

Parity status per function is stated in its docstring; the pins live in
tests/test_oracle_*.py.
"""
import math

import numpy as np

U64 = np.uint64
M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15

KIND_PAGE = 0
KIND_HEAD = 1
KIND_SIGN = 2

HASH_VERSION = 1


# ----------------------------------------------------------------------------
# splitmix64 (Steele, Lea, Flood, OOPSLA 2014), written from its definition


def mix64(z):
    """splitmix64's output function on a uint64 array, wrapping arithmetic."""
    z = np.array(z, dtype=U64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> U64(30)
        z *= U64(0xBF58476D1CE4E5B9)
        z ^= z >> U64(27)
        z *= U64(0x94D049BB133111EB)
        z ^= z >> U64(31)
    return z


def splitmix64(seed, i):
    """Output i (0-based) of splitmix64 whose state starts at ``seed``.

    The state after i+1 steps is seed + (i+1)*0x9E3779B97F4A7C15 (mod 2^64);
    the output is mix64 of that state.
    """
    state = (int(seed) + (int(i) + 1) * GOLDEN) & M64
    return int(mix64(np.array([state], dtype=U64))[0])


# ----------------------------------------------------------------------------
# Hash constants and the multiply-XOR hash


def role_index(n, kind, k=0, w=0):
    """Flat index of a hash role: page hash b_n, head hash u_{n,k}, or sign
    word w of head (n,k). Independent of K and r, so two layouts that share
    a hash seed share every hash function."""
    assert 0 <= n < 8 and 0 <= kind < 4 and 0 <= k < 64 and 0 <= w < 8
    return ((n * 4 + kind) * 64 + k) * 8 + w


def role_constants(seed, n, kind, k=0, w=0):
    """Seed word c and odd multipliers a_0..a_{n-1} of one hash role.

    Reading of the Engram notes §3.2 ("a lightweight multiply-XOR hash"), which
    give no constants: c = output 8*idx of the hash seed's splitmix64 stream,
    a_j = output 8*idx+1+j with the low bit forced to 1.
    """
    idx = role_index(n, kind, k, w)
    c = splitmix64(seed, 8 * idx)
    a = [splitmix64(seed, 8 * idx + 1 + j) | 1 for j in range(n)]
    return c, a


def ngram_hash(g, c, a):
    """Multiply-XOR hash of n-grams ``g`` (uint64 [..., n], g[...,j] is the
    canonical ID at position t-j): mix64(c XOR a_0*g_0 XOR ... XOR a_{n-1}*g_{n-1}),
    products taken mod 2^64 (Engram notes §3.2, multiply-XOR hashing; the
    splitmix64 finaliser is the reading that makes slots of different heads
    independent, which the collision pins check)."""
    g = np.asarray(g, dtype=U64)
    x = np.full(g.shape[:-1], c, dtype=U64)
    with np.errstate(over="ignore"):
        for j in range(g.shape[-1]):
            x ^= g[..., j] * U64(a[j])
    return mix64(x)


# ----------------------------------------------------------------------------
# Steps 1-2: canonical IDs and suffix n-grams


def canonicalize(tokens, canon_map, pad_id):
    """c = P(x) for each token (Engram notes §3.2, tokenizer compression:
    a precomputed surjection V -> V'). Token IDs outside [0, V) become PAD;
    the second return value says whether any did."""
    tokens = np.asarray(tokens, dtype=np.int64)
    cmap = np.asarray(canon_map, dtype=np.int64)
    V = cmap.shape[0]
    ok = (tokens >= 0) & (tokens < V)
    c = np.where(ok, cmap[np.clip(tokens, 0, max(V - 1, 0))] if V else 0,
                 pad_id)
    return c.astype(np.int64), bool((~ok).any())


def suffix_ngrams(canon, n, pad_id):
    """g_{t,n} = (c_{t-n+1}, ..., c_t) per sequence (Engram notes §3.2; PageGram
    §2.1), stored newest first: out[b, t, j] = c[b, t-j], PAD where t-j < 0.
    Rows of [B, T] are separate sequences; nothing crosses them."""
    canon = np.asarray(canon, dtype=np.int64)
    B, T = canon.shape
    g = np.full((B, T, n), pad_id, dtype=np.int64)
    for j in range(n):
        if j < T:
            g[:, j:, j] = canon[:, :T - j]
    return g


# ----------------------------------------------------------------------------
# Steps 3-4: hashes and rows


def layout_orders(layout):
    return list(range(layout["n_min"], layout["n_max"] + 1))


def sign_words_per_head(layout):
    return (layout["r"] + 63) // 64


def layout_bases(layout):
    """Row bases and the total row count R of one table T in R^{R x r}.

    PageGram §3.1: each order n owns P_n pages of K*S rows; order bases are
    cumulative (order 2 first). Engram-style (PageGram §2.2): head (n,k) owns
    a sub-table of P_{n,k} rows; bases are cumulative in (n, k) order."""
    K, S = layout["K"], layout["S"]
    orders = layout_orders(layout)
    if layout["kind"] == "pagegram":
        bases, acc = [], 0
        for i, _ in enumerate(orders):
            bases.append(acc)
            acc += int(layout["pages"][i]) * K * S
        return bases, acc
    bases, acc = [], 0
    for i, _ in enumerate(orders):
        row = []
        for k in range(K):
            row.append(acc)
            acc += int(layout["head_rows"][i * K + k])
        bases.append(row)
    return bases, acc


def index(layout, tokens, canon_map, pad_id):
    """Canonical IDs, hashes, rows, pages and sign words for every token.

    Returns a dict with (N = B*T, O = number of orders, W = ceil(r/64)):
      canon  int64 [B, T]
      hashes uint64 [N, O, 1+K]   (b_n, u_{n,0}, ..., u_{n,K-1})
      rows   int64 [N, O, K]
      pages  int64 [N, O]         (p_n; -1 for the Engram-style layout)
      signs  uint64 [N, O, K, W]  (0 when signs are off)
      bad    bool                 (a token was outside [0, V))

    PageGram §3.1: p_n = b_n mod P_n and
        row_{n,k} = base_n + (p_n K + k) S + (u_{n,k} mod S).
    PageGram §2.2 (Engram-style): row_{n,k} = base_{n,k} + u_{n,k} mod P_{n,k}.
    Signs: PageGram §2.1 and §3.1, hash-generated pseudo-random +-1 vectors.
    """
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    N = B * T
    K, S = layout["K"], layout["S"]
    seed = layout["hash_seed"]
    orders = layout_orders(layout)
    O = len(orders)
    Wd = sign_words_per_head(layout)
    canon, bad = canonicalize(tokens, canon_map, pad_id)
    bases, _ = layout_bases(layout)

    hashes = np.zeros((N, O, 1 + K), dtype=U64)
    rows = np.zeros((N, O, K), dtype=np.int64)
    pages = np.full((N, O), -1, dtype=np.int64)
    signs = np.zeros((N, O, K, Wd), dtype=U64)
    for i, n in enumerate(orders):
        g = suffix_ngrams(canon, n, pad_id).reshape(N, n)
        c, a = role_constants(seed, n, KIND_PAGE)
        b = ngram_hash(g, c, a)
        hashes[:, i, 0] = b
        if layout["kind"] == "pagegram":
            P = U64(layout["pages"][i])
            p = (b % P).astype(np.int64)
            pages[:, i] = p
        for k in range(K):
            c, a = role_constants(seed, n, KIND_HEAD, k)
            u = ngram_hash(g, c, a)
            hashes[:, i, 1 + k] = u
            if layout["kind"] == "pagegram":
                slot = (u % U64(S)).astype(np.int64)
                rows[:, i, k] = bases[i] + (p * K + k) * S + slot
            else:
                Pk = U64(layout["head_rows"][i * K + k])
                rows[:, i, k] = bases[i][k] + (u % Pk).astype(np.int64)
            if layout["use_signs"]:
                for w in range(Wd):
                    c, a = role_constants(seed, n, KIND_SIGN, k, w)
                    signs[:, i, k, w] = ngram_hash(g, c, a)
    return dict(canon=canon, hashes=hashes, rows=rows, pages=pages,
                signs=signs, bad=bad)


def sign_vectors(signs, r):
    """+-1 vectors from sign words: element j -> bit j%64 of word j//64,
    bit set -> -1. ``signs`` uint64 [..., W] -> float64 [..., r]."""
    signs = np.asarray(signs, dtype=U64)
    j = np.arange(r)
    bits = (signs[..., j // 64] >> (j % 64).astype(U64)) & U64(1)
    return 1.0 - 2.0 * bits.astype(np.float64)


# ----------------------------------------------------------------------------
# NF4 format (PageGram §2.3 and §3.3: 64 4-bit codes plus one fp16 scale per
# row; QLoRA's NormalFloat codebook)


def nf4_codebook():
    """The 16 NF4 levels as fp32 values, ascending.

    QLoRA's NormalFloat construction: quantiles of the standard normal,
    asymmetric (8 positive levels, 7 negative ones and an exact zero) and
    normalised to [-1, 1]. Reading: the outermost quantile is taken at
    probability delta = ((1 - 1/30) + (1 - 1/32)) / 2, halfway between the
    outer positions of 15 and 16 evenly spaced levels; positive levels sit at
    linspace(delta, 1/2, 9) without its last point, negative ones at
    linspace(delta, 1/2, 8) without its last point, mirrored. Parity with
    QLoRA's printed table: unpinned (not on the pages).
    """
    from scipy.stats import norm
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    pos = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    v = v / np.max(np.abs(v))
    return v.astype(np.float32)


def nf4_unpack(codes, r):
    """uint8 [..., r/2] -> int codes [..., r]; code j sits in byte j>>1,
    low nibble for even j."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes & 0x0F
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (r,), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def nf4_dequantize(codes, scales, r):
    """Exact dequantised values (float64): codebook[code] * scale."""
    cb = nf4_codebook().astype(np.float64)
    q = nf4_unpack(codes, r)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    return cb[q] * s[..., None]


def nf4_quantize(x):
    """Per-row absmax NF4 quantisation of float rows [n, r] (export side).

    scale = fp16(max |x|); code = nearest codebook level to x/scale. An
    all-zero row gets scale 0 and the zero code, so it dequantises to exact
    zeros (PageGram §9.4, check 5)."""
    x = np.asarray(x, dtype=np.float64)
    n, r = x.shape
    cb = nf4_codebook().astype(np.float64)
    absmax = np.max(np.abs(x), axis=1)
    scale = absmax.astype(np.float16)
    s64 = scale.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(s64[:, None] > 0, x / s64[:, None], 0.0)
    q = np.argmin(np.abs(y[..., None] - cb[None, None, :]), axis=-1)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale


# ----------------------------------------------------------------------------
# Step 5: gather, dequantise, sign, concatenate


def _rows_as_f64(table_dtype, stored, r):
    if table_dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if table_dtype == "bf16":
        b = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    if table_dtype == "nf4":
        codes, scales = stored
        return nf4_dequantize(codes, scales, r)
    raise ValueError(table_dtype)


def gather(layout, table_dtype, fetch, rows, signs):
    """e_t = concat over n (outer) and k (inner) of s_{n,k} * deq(T[row_{n,k}])
    (PageGram §2.2 and §3.1; Engram notes §3.2, concatenation order n then k).

    ``fetch(rows_flat)`` returns the stored values of those table rows (f32,
    bf16 bit patterns, or (codes, scales) for NF4). Returns float64 [N, O*K*r].
    """
    r = layout["r"]
    rows = np.asarray(rows, dtype=np.int64)
    N, O, K = rows.shape
    vals = _rows_as_f64(table_dtype, fetch(rows.reshape(-1)), r)
    vals = vals.reshape(N, O, K, r)
    if layout["use_signs"]:
        vals = vals * sign_vectors(signs, r)
    return vals.reshape(N, O * K * r)


def _f32_to_bf16_bits(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    return ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def gather_stored(layout, table_dtype, fetch, rows, signs):
    """The concatenated e in the precision it is stored in on the device:
    float32 for an fp32 table, bf16 bit patterns (uint16) otherwise.

    fp32 / bf16 tables: the stored value with its sign flipped, exactly.
    NF4: fp32(codebook[code] * fp32(scale)) rounded to nearest even, sign
    applied, then rounded to bf16 (nearest even). Used for bit-exact checks.
    """
    r = layout["r"]
    rows = np.asarray(rows, dtype=np.int64)
    N, O, K = rows.shape
    stored = fetch(rows.reshape(-1))
    sg = (sign_vectors(signs, r) if layout["use_signs"]
          else np.ones((N, O, K, r)))
    neg = (sg < 0).reshape(N * O * K, r)
    if table_dtype == "f32":
        v = np.asarray(stored, dtype=np.float32).reshape(N * O * K, r).copy()
        v[neg] = -v[neg]
        return v.reshape(N, O * K * r)
    if table_dtype == "bf16":
        v = np.asarray(stored, dtype=np.uint16).reshape(N * O * K, r).copy()
        v[neg] ^= np.uint16(0x8000)
        return v.reshape(N, O * K * r)
    codes, scales = stored
    cb = nf4_codebook()
    q = nf4_unpack(codes, r)
    prod = cb[q] * np.asarray(scales, dtype=np.float16).astype(np.float32)[:, None]
    prod = prod.astype(np.float32)
    prod[neg] = -prod[neg]
    return _f32_to_bf16_bits(prod).reshape(N, O * K * r)


# ----------------------------------------------------------------------------
# Steps 6-7: projection and fusion into the residual stream


def project(e, W):
    """y = W e for each token (PageGram §2.2: W_V in R^{d x 2Kr}); W row-major
    [d_out, E] as stored; float64."""
    return np.asarray(e, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def scalar_gate(x, y, g):
    """x <- x + g e_t with a per-layer scalar gate (PageGram §3.1). ``x`` may
    be None, in which case the increment g*y alone is returned."""
    inc = float(g) * np.asarray(y, dtype=np.float64)
    if x is None:
        return inc
    return np.asarray(x, dtype=np.float64) + inc


def rmsnorm(x, gamma, eps):
    """RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def causal_dwconv_at(z_of, t, w, dil):
    """Causal depthwise conv output at position t of one sequence:
    y_t[c] = sum_j w[c, j] * z_{t - (kw-1-j)*dil}[c], zero before the start
    (torch conv1d cross-correlation with left zero padding, groups = d;
    Engram notes §3.3, kernel 4, dilation = max n-gram order).
    ``z_of(tau)`` returns z at position tau >= 0."""
    kw = w.shape[1]
    y = np.zeros(w.shape[0], dtype=np.float64)
    for j in range(kw):
        tau = t - (kw - 1 - j) * dil
        if tau >= 0:
            y += w[:, j] * z_of(tau)
    return y


def engram_gate_fusion(h, e_of, W, d, M, gamma_h, gamma_k, gamma_u, conv_w,
                       dil, eps, positions, T):
    """Engram fusion increment Y^m at the requested positions.

    For branch m (Engram notes §3.3-3.4; Engram explainer, gate formulas):
      v = W_V e, k^m = W_K^(m) e,
      alpha^m = sigmoid(RMSNorm(h^m) . RMSNorm(k^m) / sqrt(d)),
      u~^m = alpha^m v,
      Y^m = SiLU(CausalDWConv(RMSNorm(u~^m))) + u~^m.
    W is [(1+M) d, E] = [W_V; W_K^(1); ...; W_K^(M)]. ``h`` is a callable:
    h(m, flat) returns the hidden row h^m at flat position flat = b*T + t;
    e_of(flat) returns e there.
    ``positions`` are flat positions; returns float64 [M, len(positions), d].
    """
    W = np.asarray(W, dtype=np.float64)
    Wv = W[:d]
    cache = {}

    def fused_at(flat):
        if flat not in cache:
            e = np.asarray(e_of(flat), dtype=np.float64)
            v = Wv @ e
            us = []
            for m in range(M):
                k = W[d * (1 + m):d * (2 + m)] @ e
                hn = rmsnorm(h(m, flat), gamma_h, eps)
                kn = rmsnorm(k, gamma_k, eps)
                alpha = sigmoid(np.dot(hn, kn) / math.sqrt(d))
                us.append(alpha * v)
            cache[flat] = us
        return cache[flat]

    out = np.zeros((M, len(positions), d), dtype=np.float64)
    for i, flat in enumerate(positions):
        b, t = divmod(int(flat), T)
        for m in range(M):
            z_of = (lambda tau, m=m: rmsnorm(fused_at(b * T + tau)[m],
                                             gamma_u, eps))
            conv = causal_dwconv_at(z_of, t, np.asarray(conv_w, np.float64), dil)
            out[m, i] = silu(conv) + fused_at(flat)[m]
    return out


# ----------------------------------------------------------------------------
# Whole path


def forward_scalar(layout, pad_id, tokens, canon_map, table_dtype, fetch, W,
                   g, x, positions=None):
    """Scalar-gated path at the given flat positions (all when None).

    ``x`` is None (increment only) or a callable x(flat_positions) returning
    the residual rows. Returns dict(index, positions, e, y, out)."""
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    idx = index(layout, tokens, canon_map, pad_id)
    pos = (np.arange(B * T) if positions is None
           else np.asarray(positions, dtype=np.int64))
    e = gather(layout, table_dtype, fetch, idx["rows"][pos], idx["signs"][pos])
    y = project(e, W)
    out = scalar_gate(None if x is None else x(pos), y, g)
    return dict(index=idx, positions=pos, e=e, y=y, out=out)


def forward_engram(layout, pad_id, tokens, canon_map, table_dtype, fetch, W,
                   d, M, gamma_h, gamma_k, gamma_u, conv_w, dil, eps, h,
                   positions=None, with_resid=True):
    """Engram-fusion path at the given flat positions (all when None).

    ``h(m, flat)`` returns h^m at a flat position. Returns dict(index,
    positions, out) with out float64 [M, len(positions), d]: h^m + Y^m, or
    Y^m alone when with_resid is False (Engram notes §3.1: H <- H + Y)."""
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    idx = index(layout, tokens, canon_map, pad_id)
    pos = (np.arange(B * T) if positions is None
           else np.asarray(positions, dtype=np.int64))
    rows, signs = idx["rows"], idx["signs"]

    def e_of(flat):
        return gather(layout, table_dtype, fetch, rows[flat:flat + 1],
                      signs[flat:flat + 1])[0]

    Y = engram_gate_fusion(h, e_of, W, d, M, gamma_h, gamma_k, gamma_u, conv_w,
                           dil, eps, pos, T)
    if with_resid:
        Y = Y + np.stack([np.stack([np.asarray(h(m, int(f)), np.float64)
                                    for f in pos]) if len(pos) else
                          np.zeros((0, d)) for m in range(M)])
    return dict(index=idx, positions=pos, out=Y)
