"""The five synthetic workloads the hot path is tested and measured on.

Each workload is a plain dict of sizes, distributions and seeds: the n-gram
memory layout (orders 2 and 3, K heads, S slots, row width r, page counts or
per-head prime sizes), the token stream, the table and projection
distributions and the fusion stage. Nothing here computes any part of the
method; the per-head prime sizes of the Engram-style layouts are written out
as literals (their primality is checked by the oracle's tests).

Sources (PageGram tech report, Empero AI, 2026-10; Engram notes on
"Conditional Memory via Scalable Lookup", arXiv 2601.07372):
  * orders {2,3}, K=8, r=64, 200M-parameter tables, S=4 -- PageGram §4
    (external table configuration);
  * per-head prime sizes near 195,300 for the Engram-style comparison --
    PageGram §4 and §2.2;
  * 4-bit rows of 64 codes plus an fp16 scale -- PageGram §2.3, §3.3;
  * 128k vocabulary compressed by about 23% -- Engram notes §3.2;
  * Engram-27B: 8 heads, memory dimension 1280, hidden 2560, M=4 branches,
    5.7B-parameter table, conv kernel 4 with dilation 3 -- Engram notes §3.3,
    §3.4, §3.7.
"""

HASH_SEED = 0x5EED0001

# First 16 primes >= 195,313 (= 200M / (16 * 64)), ascending; assigned to
# (n=2, k=0..7) then (n=3, k=0..7).
ENGRAM_200M_PRIMES = [
    195319, 195329, 195341, 195343, 195353, 195359, 195389, 195401,
    195407, 195413, 195427, 195443, 195457, 195469, 195479, 195493,
]
# First 16 primes >= 4,453,125 (= 5.7B / (16 * 80)), same assignment order.
ENGRAM_27B_PRIMES = [
    4453129, 4453139, 4453147, 4453159, 4453171, 4453177, 4453187, 4453213,
    4453223, 4453231, 4453259, 4453271, 4453291, 4453321, 4453331, 4453349,
]

# Engram-style comparison layout for the 20B NF4 table: the first 16 primes
# >= 312,500,000 / 16 (the page-cache comparison of PageGram §8 at equal size).
ENGRAM_20B_PRIMES = [
    19531261, 19531289, 19531327, 19531339, 19531381, 19531387, 19531403, 19531409,
    19531423, 19531433, 19531441, 19531493, 19531517, 19531541, 19531543, 19531553,
]

# Stream identifiers of the counter-based value generator (synth.gen).
STREAM_TABLE = 1
STREAM_NF4_SCALE = 2
STREAM_W = 3
STREAM_RESID = 4
STREAM_GAMMA_H = 5
STREAM_GAMMA_K = 6
STREAM_GAMMA_U = 7
STREAM_CONV = 8


def _layout(kind, K, S, r, pages=None, primes=None, use_signs=1):
    return dict(kind=kind, n_min=2, n_max=3, K=K, S=S, r=r,
                pages=list(pages or []), head_rows=list(primes or []),
                hash_seed=HASH_SEED, use_signs=use_signs)


WORKLOADS = {
    # Tiny fp32 case: small enough for element-wise oracle checks everywhere.
    "tiny_pagegram_fp32_1x256": dict(
        layout=_layout("pagegram", K=4, S=4, r=16, pages=[64, 64]),
        vocab=1024, canon_vocab=1024, canon="identity", map_seed=1,
        B=1, T=256, token_dist="uniform", token_seed=1,
        table_dtype="f32", table_sigma=0.02, table_seed=1,
        act_dtype="f32", d=64, w_sigma=0.05, resid_sigma=1.0,
        gate="scalar", g=0.5, data_seed=1,
    ),
    # PageGram 200M-parameter bf16 table: the headline throughput workload.
    "pagegram200m_bf16_8x2048": dict(
        layout=_layout("pagegram", K=8, S=4, r=64, pages=[48828, 48828]),
        vocab=50304, canon_vocab=50304, canon="identity", map_seed=2,
        B=8, T=2048, token_dist="zipf", zipf_s=1.1, token_seed=2,
        table_dtype="bf16", table_sigma=0.02, table_seed=2,
        act_dtype="bf16", d=768, w_sigma=0.05, resid_sigma=1.0,
        gate="scalar", g=0.5, data_seed=2,
    ),
    # Engram-style per-head prime tables at the same parameter count and the
    # same token stream, projection, gate and hash functions.
    "engram200m_bf16_8x2048": dict(
        layout=_layout("engram", K=8, S=1, r=64, primes=ENGRAM_200M_PRIMES),
        vocab=50304, canon_vocab=50304, canon="identity", map_seed=2,
        B=8, T=2048, token_dist="zipf", zipf_s=1.1, token_seed=2,
        table_dtype="bf16", table_sigma=0.02, table_seed=2,
        act_dtype="bf16", d=768, w_sigma=0.05, resid_sigma=1.0,
        gate="scalar", g=0.5, data_seed=2,
    ),
    # NF4 20B-parameter PageGram table, 312.5M rows of 34 bytes.
    "pagegram20b_nf4_16x4096": dict(
        layout=_layout("pagegram", K=8, S=4, r=64,
                       pages=[4882812, 4882812]),
        vocab=128000, canon_vocab=98000, canon="surjective", map_seed=4,
        B=16, T=4096, token_dist="zipf", zipf_s=1.1, token_seed=4,
        table_dtype="nf4", table_sigma=0.02, table_seed=4,
        act_dtype="bf16", d=2560, w_sigma=0.05, resid_sigma=1.0,
        gate="scalar", g=0.5, data_seed=4,
    ),
    # Engram-27B-style fusion layer: one GEMM over [W_V; W_K^(1..4)], context
    # gate, RMSNorm, causal depthwise conv (kernel 4, dilation 3), SiLU, skip.
    "engram27b_fusion_bf16_32x4096": dict(
        layout=_layout("engram", K=8, S=1, r=80, primes=ENGRAM_27B_PRIMES),
        vocab=128000, canon_vocab=98000, canon="surjective", map_seed=4,
        B=32, T=4096, token_dist="zipf", zipf_s=1.1, token_seed=5,
        table_dtype="bf16", table_sigma=0.02, table_seed=5,
        act_dtype="bf16", d=2560, w_sigma=0.05, resid_sigma=1.0,
        gate="engram", M=4, eps=1e-6, conv_k=4, conv_dil=3,
        conv_sigma=0.5, gamma="ones", data_seed=5,
    ),
    # The 20B NF4 table at S = 15: a page of K*S = 120 NF4 head rows is
    # 120 * 34 = 4080 bytes, one 4 KiB block (PageGram §3.3); P_n chosen so the
    # table keeps the 20B workload's 156.25M rows per order (1,302,083 pages).
    "pagegram20b_nf4_s15_16x4096": dict(
        layout=_layout("pagegram", K=8, S=15, r=64,
                       pages=[1302083, 1302083]),
        vocab=128000, canon_vocab=98000, canon="surjective", map_seed=4,
        B=16, T=4096, token_dist="zipf", zipf_s=1.1, token_seed=4,
        table_dtype="nf4", table_sigma=0.02, table_seed=6,
        act_dtype="bf16", d=2560, w_sigma=0.05, resid_sigma=1.0,
        gate="scalar", g=0.5, data_seed=4,
    ),
    # The same 20B NF4 table in the Engram-style layout (16 prime head tables,
    # 312,502,740 rows): the comparison side of the flash page-cache figures.
    "engram20b_nf4_16x4096": dict(
        layout=_layout("engram", K=8, S=1, r=64, primes=ENGRAM_20B_PRIMES),
        vocab=128000, canon_vocab=98000, canon="surjective", map_seed=4,
        B=16, T=4096, token_dist="zipf", zipf_s=1.1, token_seed=4,
        table_dtype="nf4", table_sigma=0.02, table_seed=7,
        act_dtype="bf16", d=2560, w_sigma=0.05, resid_sigma=1.0,
        gate="scalar", g=0.5, data_seed=4,
    ),
}

# Order used when a workload is referred to by position.
ORDER = list(WORKLOADS)


def workload(name_or_index):
    """Return a copy of a workload dict, by name or by position in ORDER."""
    if isinstance(name_or_index, int):
        name_or_index = ORDER[name_or_index]
    wl = dict(WORKLOADS[name_or_index])
    wl["name"] = name_or_index
    wl["layout"] = dict(wl["layout"])
    return wl


def with_tokens(wl, B, T):
    """Same workload with a different batch shape (for parity cases)."""
    out = dict(wl)
    out["layout"] = dict(wl["layout"])
    out["B"], out["T"] = int(B), int(T)
    return out


def e_dim(wl):
    lay = wl["layout"]
    return (lay["n_max"] - lay["n_min"] + 1) * lay["K"] * lay["r"]


def d_out(wl):
    return wl["d"] * (1 + wl["M"]) if wl["gate"] == "engram" else wl["d"]
