"""Throughput of the n-gram memory hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--only]
                    [--no-cpu-baseline] [--no-cold] [--fp8]

A step is one pg_forward call over one batch of synthetic tokens: canonical
map, n-grams, hashes, rows, gather/dequant/sign, concatenation, projection
and fusion. Steps cycle through a pool of 32 distinct token batches already
resident in HBM, so the table rows of one step are not left in the caches by
the previous one.

The headline workload is the largest one that fits one GPU: the Engram-27B
style fusion layer (32 x 4096 tokens, 5.7B-parameter bf16 table, the fused
[W_V; W_K^(1..4)] projection of 12,800 x 1,280, context gate and causal
conv). Its timed region is K steps back to back (wall clock for the value;
a HIP event before each step for the median, p10 and p90), after a warm-up
of at least W steps and at least one second. Each kernel's launch durations
are then measured alone, K launches of its entry point between HIP events on
the stream it runs on (pg_index_gather, pg_engram_project, pg_engram_gate,
pg_engram_mix for the Engram workload; pg_forward is checked bit for bit
against them). A cold variant times single steps after a 1 GiB device write
that evicts the caches (the write is outside the timed interval).

The other workloads (the 200M PageGram and Engram-style tables and the 20B
NF4 table) follow as extra keys with the same per-kernel figures, fewer
steps and no cold variant (--only skips them).

Prints one JSON line: whole-job tokens/s, the roofline position of the
dominant kernel (algorithmic flops or bytes per launch over its mean launch
duration), every kernel's figures, the measured streaming-read rate of the
GPU, and the CPU oracle timed on a bounded sample on the host cores.

--fp8 times the same path with E4M3 projection operands instead (W
quantised once before timing): a separate line at another precision, never
the headline.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector
POOL = 32
DEFAULT_WORKLOAD = "engram27b_fusion_bf16_32x4096"
BACKWARD_WORKLOAD = "pagegram200m_bf16_8x2048"   # the backward needs the scalar gate
HOST_TABLE_WORKLOAD = "pagegram200m_bf16_8x2048"  # so does the host-table step
SECONDARY = ["pagegram200m_bf16_8x2048", "engram200m_bf16_8x2048", "pagegram20b_nf4_16x4096"]
SECONDARY_STEPS = 200           # timed steps of the extra workloads (at most)
WARM_S = 1.0                    # seconds of untimed steps before the headline timing
WARM_S_SECONDARY = 0.3
COLD_STEPS = 20                 # single steps after a cache-evicting write
FLUSH_BYTES = 1 << 30
READ_PROBE_BYTES = 4 << 30
# E4M3 scale exponents of the --fp8 mode: e ~ N(0, 0.02) rows (NF4: |e| <=
# about 0.05) and W ~ N(0, 0.05) times 2^s stay well below 448
FP8_E_SCALE = {"bf16": 11, "nf4": 13, "f32": 11}
FP8_W_SCALE = 10


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20,
                   help="untimed steps before timing (and at least one second of them)")
    p.add_argument("--workload", default=None,
                   help=f"workload name (default {DEFAULT_WORKLOAD}; {BACKWARD_WORKLOAD} "
                        f"with --backward, {HOST_TABLE_WORKLOAD} with --host-table)")
    p.add_argument("--only", action="store_true", help="the headline workload alone")
    p.add_argument("--no-cold", action="store_true", help="skip the cache-evicted variant")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=None,
                   help="tokens per oracle batch (default: one sequence, at most 16,384)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a 1 GiB device copy (for counter scaling)")
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (pg_backward_scalar) and the row-wise RMS "
                        "table update (pg_row_rms_step) on the workload")
    p.add_argument("--page-cache", action="store_true",
                   help="flash page-cache figures (reads/token under an LRU RAM cache) "
                        "of the 20B NF4 table in the PageGram S=4, S=15 and Engram-style "
                        "layouts, from pg_index rows of the token pool")
    p.add_argument("--host-table", action="store_true",
                   help="table in pinned host memory: pg_index, pg_stage_rows (touched units "
                        "to an HBM cache), pg_gather_staged, pg_project_gate per step, "
                        "sequential and with the next step's staging on a second stream")
    p.add_argument("--stage-unit", choices=["page", "row"], default="page",
                   help="--host-table unit of transfer: pages / 4 KiB runs, or single rows")
    p.add_argument("--fp8", action="store_true",
                   help="E4M3 projection operands (pg_forward_fp8); a separate line")
    p.add_argument("--traffic-from", nargs="+", metavar="CSV",
                   help="write profiles/traffic.json from rocprofv3 --pmc counter "
                        "collections of --copy-probe runs: FETCH_SIZE, WRITE_SIZE and "
                        "optionally TCC_EA0_RDREQ{,_32B,_64B,_128B}_sum (read requests "
                        "by size)")
    a = p.parse_args()
    if a.workload is None:
        a.workload = (BACKWARD_WORKLOAD if a.backward else
                      HOST_TABLE_WORKLOAD if a.host_table else DEFAULT_WORKLOAD)
    return a


def algorithmic_costs(wl, fp8=False):
    """Per-token algorithmic HBM bytes of index+gather and flops/bytes of the
    projection stage (the figures the roofline uses). fp8: e is one byte per
    element (residual and output stay bf16)."""
    lay = wl["layout"]
    O = lay["n_max"] - lay["n_min"] + 1
    K, r = lay["K"], lay["r"]
    elt = 4 if wl["act_dtype"] == "f32" else 2
    e_elt = 1 if fp8 else elt
    row_bytes = {"f32": 4 * r, "bf16": 2 * r, "nf4": r // 2 + 2}[wl["table_dtype"]]
    E = O * K * r
    gather_bytes = 4 + O * K * row_bytes + E * e_elt
    extra = {}
    if wl["gate"] == "engram":
        M, d = wl["M"], wl["d"]
        n_cb = d // 256
        flops = 2 * E * (1 + M) * d
        proj_bytes = E * e_elt + 2 * M * d * elt   # e in; h in, out (pass 1 + 2 read h)
        # pass 1: e and h in; v and the partial sums (sum v^2; per branch
        # sum k^2, sum gamma_h gamma_k h k, sum h^2 per 256 columns) out.
        # pass 2: h and v in, out out (the gates are 8 M bytes per token).
        extra = dict(pass1_bytes=E * e_elt + M * d * elt + d * elt + 4 * n_cb * (1 + 3 * M),
                     pass2_bytes=2 * M * d * elt + d * elt + 8 * M)
    else:
        d = wl["d"]
        flops = 2 * E * d
        proj_bytes = E * e_elt + 2 * d * elt       # e in; x in, out
    return dict(gather_bytes=gather_bytes, proj_flops=flops, proj_bytes=proj_bytes, E=E,
                **extra)


def code_text(text):
    """A kernel source's code: // comments, trailing blanks and empty lines
    dropped (the sources have no /* */ comments and no // inside strings), so
    that counters taken on a kernel stay attached to it when only its
    comments change."""
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gather": ["hashed_head_gram_amd/csrc/index.hip", "hashed_head_gram_amd/csrc/common.h"],
    "projection": ["hashed_head_gram_amd/csrc/gemm.hip", "hashed_head_gram_amd/csrc/common.h"],
    "gathered": ["hashed_head_gram_amd/csrc/gemm.hip", "hashed_head_gram_amd/csrc/common.h"],
    "pass1": ["hashed_head_gram_amd/csrc/gemm_slots.hip", "hashed_head_gram_amd/csrc/common.h"],
    "pass2": ["hashed_head_gram_amd/csrc/engram.hip", "hashed_head_gram_amd/csrc/common.h"],
}


def traffic_for(stage, workload):
    """HBM bytes per launch from committed counter runs, if the kernel source
    is unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(stage)
    if not ent or ent.get("source_digest") != source_digest(KERNEL_SOURCES[stage]):
        return None
    return ent.get("bytes_per_launch")


COPY_BYTES = 1 << 30
COPY_REPS = 5
TRAFFIC_KERNELS = {"gather": "index_gather_kernel", "projection": "gemm_pipe_kernel",
                   "gathered": "gemm_pipe_gather_kernel", "pass1": "engram_slot_kernel",
                   "pass2": "engram_pass2_kernel",
                   "copy": "copyBuffer"}


def counter_means(path, counter):
    """Mean per-dispatch value of one counter for each kernel family (KiB for
    FETCH_SIZE and WRITE_SIZE, requests for the TCC_EA0_RDREQ family)."""
    import csv
    sums = {}
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] not in (counter, counter + "_sum"):
            continue
        for fam, key in TRAFFIC_KERNELS.items():
            if key in row["Kernel_Name"]:
                d = sums.setdefault(fam, {})
                d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    # the copy family: only the 1 GiB probe copies, the last COPY_REPS copies
    # of the run (set-up copies of other sizes, some larger, come before them)
    if "copy" in sums:
        last = sorted(sums["copy"], key=int)[-COPY_REPS:]
        sums["copy"] = {k: sums["copy"][k] for k in last}
    return {fam: sum(d.values()) / len(d) for fam, d in sums.items() if d}


def read_bytes_by_size(rdreq_csv):
    """Bytes read from HBM per dispatch and family from the memory-side read
    requests counted by size (32, 64 and 128 bytes; requests of none of the
    three sizes, if any, taken as 64 bytes)."""
    n = {sz: counter_means(rdreq_csv, "TCC_EA0_RDREQ" + sz) for sz in ("", "_32B", "_64B", "_128B")}
    out = {}
    for fam, tot in n[""].items():
        r32, r64, r128 = (n[sz].get(fam, 0.0) for sz in ("_32B", "_64B", "_128B"))
        other = max(tot - r32 - r64 - r128, 0.0)
        out[fam] = {"bytes": 32 * r32 + 64 * (r64 + other) + 128 * r128, "req": tot,
                    "req_32B": r32, "req_64B": r64, "req_128B": r128}
    return out


def write_traffic(workload, fetch_csv, write_csv, rdreq_csv=None, path=None):
    """HBM bytes per launch of the gather and projection kernels (and of the
    gathered projection where the workload runs it): FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the
    1 GiB device copy read and write exactly 1 GiB. With rdreq_csv, read bytes
    also from the read requests by size, unscaled, next to the copy's reading
    of the same counters (which should be 1 GiB). The record goes into path
    (profiles/traffic.json by default), replacing the workload's entry."""
    fetch = counter_means(fetch_csv, "FETCH_SIZE")
    write = counter_means(write_csv, "WRITE_SIZE")
    by_size = read_bytes_by_size(rdreq_csv) if rdreq_csv else {}
    f_scale = COPY_BYTES / (fetch["copy"] * 1024)
    w_scale = COPY_BYTES / (write["copy"] * 1024)
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    ent = {}
    for stage in ("gather", "projection", "gathered", "pass1", "pass2"):
        if stage not in fetch or stage not in write:
            continue
        rd = fetch[stage] * 1024 * f_scale
        wr = write[stage] * 1024 * w_scale
        key = stage
        ent[key] = {"kernel": TRAFFIC_KERNELS[stage],
                      "source_digest": source_digest(KERNEL_SOURCES[key]),
                      "fetch_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr,
                      "fetch_kib_raw": fetch[stage], "write_kib_raw": write[stage]}
        if stage in by_size:
            ent[key]["read_requests"] = by_size[stage]
    ent["copy_scale"] = {"fetch": f_scale, "write": w_scale,
                         "copy_fetch_kib_raw": fetch["copy"], "copy_write_kib_raw": write["copy"]}
    if "copy" in by_size:
        ent["copy_scale"]["copy_read_requests"] = by_size["copy"]
    rec[workload] = ent
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps({workload: ent}, indent=1))


PAGE_CACHE_LAYOUTS = ["pagegram20b_nf4_16x4096", "pagegram20b_nf4_s15_16x4096",
                      "engram20b_nf4_16x4096"]
PAGE_CACHE_MIB = [0, 16, 64, 256, 1024, 4096]


def page_cache(batches):
    """Reads/token of the 20B NF4 table under an LRU RAM page cache of 4 KiB
    blocks, for the three layouts, over `batches` batches of the token stream.
    Rows come from pg_index on the GPU; blocks and the LRU run on the host."""
    import numpy as np
    import torch

    import hashed_head_gram_amd as pg
    import synth
    from synth import configs

    dev = torch.device("cuda:0")
    res = {}
    for name in PAGE_CACHE_LAYOUTS:
        wl = configs.workload(name)
        lay_d = wl["layout"]
        layout = pg.make_layout(lay_d["kind"], lay_d["K"], lay_d["r"], S=lay_d["S"],
                                pages=lay_d["pages"], head_rows=lay_d["head_rows"],
                                hash_seed=lay_d["hash_seed"], use_signs=lay_d["use_signs"],
                                n_min=lay_d["n_min"], n_max=lay_d["n_max"],
                                pad_id=wl["canon_vocab"])
        O = lay_d["n_max"] - lay_d["n_min"] + 1
        K, W = lay_d["K"], (lay_d["r"] + 63) // 64
        cmap = torch.from_numpy(synth.canon_map(wl)).to(dev)
        blocks = []
        t0 = time.perf_counter()
        for j in range(batches):
            toks = torch.from_numpy(synth.tokens(wl, batch=j)).to(dev)
            N = toks.numel()
            rows = torch.empty(N, O, K, dtype=torch.int64, device=dev)
            signs = torch.empty(N, O, K, W, dtype=torch.int64, device=dev)
            pg.pg_index(layout, toks, cmap, rows, signs)
            blocks.append(pg.pg_flash_blocks(layout, pg.PG_NF4, rows.cpu().numpy()))
        blocks = np.concatenate([b.reshape(b.shape[0], -1) for b in blocks])
        t1 = time.perf_counter()
        per = {}
        for mib in PAGE_CACHE_MIB:
            st = pg.pg_lru_cache_sim(blocks, mib * 1024 * 1024 // 4096)
            per[f"{mib}MiB"] = st["misses"] / st["tokens"]
        t2 = time.perf_counter()
        res[name] = {"reads_per_token": per, "tokens": int(blocks.shape[0]),
                     "uncached_reads_per_token": st["distinct"] / st["tokens"],
                     "index_s": t1 - t0, "lru_s": (t2 - t1) / len(PAGE_CACHE_MIB)}
    return res


def backward_bench(args):
    """Backward pass + sparse table update of a scalar-gate workload: K
    back-to-back calls of each entry point between HIP events."""
    import numpy as np
    import torch

    import hashed_head_gram_amd as pg
    import synth
    from synth import configs, device as sdev

    dev = torch.device("cuda:0")
    wl = configs.workload(args.workload)
    lay_d = wl["layout"]
    layout = pg.make_layout(lay_d["kind"], lay_d["K"], lay_d["r"], S=lay_d["S"],
                            pages=lay_d["pages"], head_rows=lay_d["head_rows"],
                            hash_seed=lay_d["hash_seed"], use_signs=lay_d["use_signs"],
                            n_min=lay_d["n_min"], n_max=lay_d["n_max"],
                            pad_id=wl["canon_vocab"])
    R = pg.pg_layout_rows(layout)
    r, K = lay_d["r"], lay_d["K"]
    O = lay_d["n_max"] - lay_d["n_min"] + 1
    B, T = wl["B"], wl["T"]
    N, E, d = B * T, O * K * r, wl["d"]
    L = N * O * K
    tab = torch.empty(R, r, dtype=torch.bfloat16, device=dev)
    sdev.fill_normal(tab, wl["table_seed"], configs.STREAM_TABLE, wl["table_sigma"])
    table = pg.make_table(pg.PG_BF16, tab, R)
    cmap = torch.from_numpy(synth.canon_map(wl)).to(dev)
    toks = torch.from_numpy(synth.tokens(wl)).to(dev)
    W = torch.empty(d, E, dtype=torch.bfloat16, device=dev)
    sdev.fill_normal(W, wl["data_seed"], configs.STREAM_W, wl["w_sigma"])
    dy = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
    sdev.fill_normal(dy, wl["data_seed"] + 1000, configs.STREAM_RESID, 0.1)
    rows = torch.empty(N, O, K, dtype=torch.int64, device=dev)
    signs = torch.empty(N, O, K, (r + 63) // 64, dtype=torch.int64, device=dev)
    e = torch.empty(N, E, dtype=torch.bfloat16, device=dev)
    pg.pg_index(layout, toks, cmap, rows, signs)
    pg.pg_index_gather(layout, table, toks, cmap, pg.PG_BF16, e)
    f = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, d, g=wl["g"])
    ws = torch.empty(pg.pg_backward_workspace_size(layout, f, B, T), dtype=torch.uint8,
                     device=dev)
    dW = torch.empty(d, E, dtype=torch.float32, device=dev)
    de = torch.empty(N, E, dtype=torch.float32, device=dev)
    urows = torch.empty(L, dtype=torch.int64, device=dev)
    ugrad = torch.empty(L, r, dtype=torch.float32, device=dev)
    nu = torch.zeros(1, dtype=torch.int64, device=dev)
    master = torch.zeros(R, r, dtype=torch.float32, device=dev)
    vhat = torch.zeros(R, dtype=torch.float32, device=dev)
    last = torch.zeros(R, dtype=torch.int64, device=dev)

    def bwd():
        pg.pg_backward_scalar(layout, f, rows, signs, e, dy, W, B, T, dW, de, urows, ugrad,
                              nu, ws)
    step_no = [0]

    def upd():
        step_no[0] += 1
        pg.pg_row_rms_step(layout, urows, ugrad, nu, L, master, vhat, last, step_no[0],
                           1e-2, 0.95, 0.0, 1e-8)

    def per_call_ms(fn, n):
        for _ in range(args.warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    bw_ms = per_call_ms(bwd, args.steps)
    up_ms = per_call_ms(upd, args.steps)
    n_unique = int(nu.item())
    gemm_flops = 2 * 2 * N * d * E
    return {"metric": "backward + sparse table update time per step", "unit": "ms",
            "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "dtype": "bf16 operands, fp32 gradients and master table",
            "data": "synthetic (seeded Zipf tokens, counter-generated table, W and dy)",
            "config": {"workload": wl["name"], "tokens": N, "lookups": L, "d": d, "e_dim": E,
                       "table_rows": R},
            "pg_backward_scalar_ms": bw_ms, "pg_row_rms_step_ms": up_ms,
            "distinct_rows": n_unique,
            "gemm_flops": gemm_flops,
            "gemm_only_TFLOPs_if_whole_call": gemm_flops / (bw_ms / 1e3) / 1e12,
            "backward_tokens_per_s": N / ((bw_ms + up_ms) / 1e3)}


def cpu_baseline(wl, n_tok=None, min_seconds=10.0, max_batches=64):
    """The CPU oracle on successive batches of the workload's stream
    (distinct seeded batches; one sequence each by default, at most 16,384
    tokens), until about min_seconds of timed work, with BLAS on every core
    this process may run on."""
    import numpy as np

    import oracle
    import synth

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(cores)
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    T = wl["T"]
    if n_tok is None:
        n_tok = min(16384, max(T, 16384 if wl["gate"] == "scalar" else T))
    B = max(1, min(wl["B"], n_tok // T)) if n_tok >= T else 1
    Tn = T if n_tok >= T else n_tok
    cmap = synth.canon_map(wl)
    pad = wl["canon_vocab"]
    lay = wl["layout"]
    W = synth.weight(wl)
    if wl["act_dtype"] == "bf16":
        W = synth.bf16_bits_to_f32(W)
    N = B * Tn
    if wl["gate"] == "scalar":
        x = synth.resid_rows(wl, np.arange(N))
        if wl["act_dtype"] == "bf16":
            x = synth.bf16_bits_to_f32(x)
    else:
        gh, gk, gu, cw = synth.engram_params(wl)
        M, Ntot = wl["M"], wl["B"] * wl["T"]
        rows_h = np.concatenate([m * Ntot + (np.arange(B)[:, None] * T
                                             + np.arange(Tn)[None, :]).reshape(-1)
                                 for m in range(M)])
        hh = synth.bf16_bits_to_f32(synth.resid_rows(wl, rows_h)).reshape(M, N, -1)
    total, batches = 0.0, 0
    while batches < max_batches and (batches == 0 or total < min_seconds):
        toks = synth.tokens(wl, batch=batches)[:B, :Tn]
        # Materialise the touched rows first (input generation, not timed).
        idx = oracle.index(lay, toks, cmap, pad)
        uniq = np.unique(idx["rows"].reshape(-1))
        stored = synth.table_rows(wl, uniq)

        def fetch(rows, uniq=uniq, stored=stored):
            at = np.searchsorted(uniq, rows)
            if isinstance(stored, tuple):
                return stored[0][at], stored[1][at]
            return stored[at]
        t0 = time.perf_counter()
        if wl["gate"] == "scalar":
            oracle.forward_scalar(lay, pad, toks, cmap, wl["table_dtype"], fetch, W, wl["g"],
                                  lambda p: x[p])
        else:
            oracle.forward_engram(lay, pad, toks, cmap, wl["table_dtype"], fetch, W, wl["d"],
                                  M, gh, gk, gu, cw, wl["conv_dil"], wl["eps"],
                                  lambda m, f: hh[m, f])
        total += time.perf_counter() - t0
        batches += 1
    return {"value": batches * N / total / 1e6, "unit": "Mtok/s", "cores": cores,
            "blas_threads": blas, "kind": "oracle",
            "sample": f"{batches} batches of {B}x{Tn} tokens ({batches * N} tokens, the "
                      f"first batches of the seeded stream), {total:.1f} s timed; index, "
                      f"gather and the per-token fusion single-threaded numpy, float64 "
                      f"products on {blas} BLAS threads of the {cores} cores this process "
                      f"may use"}


def host_table_bench(args):
    """Scalar-gate step with the table in pinned host memory: staged bytes
    per token and tokens/s, sequential and pipelined (the next step's index
    + staging on a second stream under this step's gather + projection,
    double-buffered caches)."""
    import numpy as np
    import torch

    import hashed_head_gram_amd as pg
    import synth
    from synth import configs, device as sdev

    dev = torch.device("cuda:0")
    wl = configs.workload(args.workload)
    if wl["gate"] != "scalar" or wl["act_dtype"] != "bf16":
        sys.exit("--host-table: scalar-gate bf16 workloads")
    lay_d = wl["layout"]
    layout = pg.make_layout(lay_d["kind"], lay_d["K"], lay_d["r"], S=lay_d["S"],
                            pages=lay_d["pages"], head_rows=lay_d["head_rows"],
                            hash_seed=lay_d["hash_seed"], use_signs=lay_d["use_signs"],
                            n_min=lay_d["n_min"], n_max=lay_d["n_max"],
                            pad_id=wl["canon_vocab"])
    R = pg.pg_layout_rows(layout)
    r, K = lay_d["r"], lay_d["K"]
    O = lay_d["n_max"] - lay_d["n_min"] + 1
    B, T = wl["B"], wl["T"]
    N, E, d = B * T, O * K * r, wl["d"]
    nf4 = wl["table_dtype"] == "nf4"
    dt = pg.PG_NF4 if nf4 else pg.PG_BF16
    # table filled on the device, then kept only in pinned host memory
    if nf4:
        dc = torch.empty(R, r // 2, dtype=torch.uint8, device=dev)
        dsc = torch.empty(R, dtype=torch.float16, device=dev)
        sdev.fill_nf4_table(dc, dsc, wl["table_seed"])
        hc = torch.empty(R, r // 2, dtype=torch.uint8, pin_memory=True)
        hsc = torch.empty(R, dtype=torch.float16, pin_memory=True)
        hc.copy_(dc)
        hsc.copy_(dsc)
        del dc, dsc
        src = pg.make_table(dt, hc, R, scales=hsc)
        row_b = r // 2 + 2
    else:
        dtab = torch.empty(R, r, dtype=torch.bfloat16, device=dev)
        sdev.fill_normal(dtab, wl["table_seed"], configs.STREAM_TABLE, wl["table_sigma"])
        htab = torch.empty(R, r, dtype=torch.bfloat16, pin_memory=True)
        htab.copy_(dtab)
        del dtab
        src = pg.make_table(dt, htab, R)
        row_b = 2 * r
    torch.cuda.empty_cache()
    cmap = torch.from_numpy(synth.canon_map(wl)).to(dev)
    pool = [torch.from_numpy(synth.tokens(wl, batch=j)).to(dev) for j in range(POOL)]
    W = torch.empty(d, E, dtype=torch.bfloat16, device=dev)
    sdev.fill_normal(W, wl["data_seed"], configs.STREAM_W, wl["w_sigma"])
    x = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
    sdev.fill_normal(x, wl["data_seed"], configs.STREAM_RESID, wl["resid_sigma"])
    fuse = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, d, g=wl["g"])
    uk = pg.PG_STAGE_ROW if args.stage_unit == "row" else pg.PG_STAGE_PAGE
    U, max_units, wsb = pg.pg_stage_geometry(layout, dt, N, unit_kind=uk)

    def buffers():
        b = dict(rows=torch.empty(N, O, K, dtype=torch.int64, device=dev),
                 signs=torch.empty(N, O, K, (r + 63) // 64, dtype=torch.int64, device=dev),
                 crows=torch.empty(N, O, K, dtype=torch.int64, device=dev),
                 nu=torch.zeros(1, dtype=torch.int64, device=dev),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=dev),
                 e=torch.empty(N, E, dtype=torch.bfloat16, device=dev),
                 out=torch.empty(N, d, dtype=torch.bfloat16, device=dev))
        if nf4:
            b["cd"] = torch.empty(max_units * U, r // 2, dtype=torch.uint8, device=dev)
            b["cs"] = torch.empty(max_units * U, dtype=torch.float16, device=dev)
            b["cache"] = pg.make_table(dt, b["cd"], max_units * U, scales=b["cs"])
        else:
            b["cd"] = torch.empty(max_units * U, r, dtype=torch.bfloat16, device=dev)
            b["cache"] = pg.make_table(dt, b["cd"], max_units * U)
        return b
    bufs = [buffers(), buffers()]

    def stage(j, b, stream=None):
        pg.pg_index(layout, pool[j % POOL], cmap, b["rows"], b["signs"], stream=stream)
        pg.pg_stage_rows(layout, src, b["rows"], b["cache"], b["crows"], b["nu"], b["ws"],
                         unit_kind=uk, stream=stream)

    def compute(b, stream=None):
        pg.pg_gather_staged(layout, b["cache"], b["crows"], b["signs"], pg.PG_BF16, b["e"],
                            stream=stream)
        pg.pg_project_gate(fuse, b["e"], B, T, W, x, b["out"], stream=stream)

    # the staged path reproduces the HBM path's e (checked once)
    stage(0, bufs[0])
    compute(bufs[0])
    torch.cuda.synchronize()
    units = []
    for j in range(POOL):
        stage(j, bufs[1])
        torch.cuda.synchronize()
        units.append(int(bufs[1]["nu"].item()))
    unit_b = U * row_b
    staged_per_tok = float(np.mean(units)) * unit_b / N

    def timed(fn, n):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for j in range(n):
            fn(j)
        z.record()
        torch.cuda.synchronize()
        return a.elapsed_time(z) / n

    for j in range(args.warmup):
        stage(j, bufs[0])
        compute(bufs[0])
    seq_ms = timed(lambda j: (stage(j, bufs[0]), compute(bufs[0])), args.steps)
    stage_ms = timed(lambda j: stage(j, bufs[0]), args.steps)
    comp_ms = timed(lambda j: compute(bufs[0]), args.steps)

    s_st, s_cp = torch.cuda.Stream(), torch.cuda.Stream()
    ready = [torch.cuda.Event(), torch.cuda.Event()]
    done = [torch.cuda.Event(), torch.cuda.Event()]

    def pipelined(n):
        cur = torch.cuda.current_stream()
        s_st.wait_stream(cur)
        s_cp.wait_stream(cur)
        with torch.cuda.stream(s_st):
            stage(0, bufs[0], stream=s_st.cuda_stream)
            ready[0].record(s_st)
        for j in range(n):
            b = j % 2
            if j + 1 < n:
                with torch.cuda.stream(s_st):
                    if j >= 1:
                        s_st.wait_event(done[(j + 1) % 2])
                    stage(j + 1, bufs[(j + 1) % 2], stream=s_st.cuda_stream)
                    ready[(j + 1) % 2].record(s_st)
            with torch.cuda.stream(s_cp):
                s_cp.wait_event(ready[b])
                compute(bufs[b], stream=s_cp.cuda_stream)
                done[b].record(s_cp)
        cur.wait_stream(s_cp)
        cur.wait_stream(s_st)

    pipelined(max(args.warmup, 2))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pipelined(args.steps)
    torch.cuda.synchronize()
    pipe_ms = (time.perf_counter() - t0) / args.steps * 1e3
    return {
        "metric": "M tokens/s with the table in pinned host memory (touched units staged "
                  "to HBM each step)",
        "value": N / (pipe_ms / 1e3) / 1e6, "unit": "Mtok/s", "higher_is_better": True,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": pipe_ms,
        "dtype": "bf16", "data": "synthetic (seeded Zipf token pool, counter-generated table)",
        "config": {"workload": wl["name"], "tokens": N, "layout": lay_d["kind"],
                   "table_dtype": wl["table_dtype"], "table_bytes": R * row_b,
                   "stage_unit": args.stage_unit, "unit_rows": U, "unit_bytes": unit_b},
        "staged_units_per_step": float(np.mean(units)),
        "staged_bytes_per_token": staged_per_tok,
        "sequential_ms_per_step": seq_ms,
        "index_plus_stage_ms": stage_ms,
        "gather_plus_project_ms": comp_ms,
        "host_link_GBps": float(np.mean(units)) * unit_b / (stage_ms / 1e3) / 1e9,
        "sequential_Mtok_s": N / (seq_ms / 1e3) / 1e6,
    }


def records_graph_ms(records_call, rec, steps):
    """Per-launch GPU time of pg_index_records: `steps` launches (cycling the
    token pool) captured in one HIP graph, replayed three times; the records
    after the last replay must equal an eager launch's."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    n = max(1, min(steps, 64))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        records_call(0)
        with torch.cuda.graph(g, stream=s):
            for j in range(n):
                records_call(j)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / n
        best = t if best is None else min(best, t)
    got = rec.clone()
    records_call(n - 1)
    torch.cuda.synchronize()
    if not torch.equal(got, rec):
        raise RuntimeError("graph-replayed records differ from an eager launch's")
    return best


def pct(a, q):
    import numpy as np
    return float(np.percentile(np.asarray(a, dtype=np.float64), q))


def spread(ms):
    """mean, median, p10 and p90 of per-launch (or per-step) times in ms."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "median": pct(a, 50), "p10": pct(a, 10),
            "p90": pct(a, 90), "n": int(a.size)}


def per_launch(fn, n):
    """Launch durations of fn(j) on the current stream: the mean of n
    launches back to back between two HIP events, then n more with an event
    before each and after the last for the median, p10 and p90 (an event
    between launches adds a few microseconds to short kernels, so the mean
    comes from the bracket alone)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for j in range(n):
        fn(j)
    b.record()
    torch.cuda.synchronize()
    mean = a.elapsed_time(b) / n
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    for j in range(n):
        ev[j].record()
        fn(j)
    ev[n].record()
    torch.cuda.synchronize()
    rec = spread([ev[j].elapsed_time(ev[j + 1]) for j in range(n)])
    rec["mean"] = mean
    return rec


def warm(fn, count, seconds):
    """At least `count` calls and at least `seconds` of wall clock (the GPU
    reaches its steady clocks before anything is timed)."""
    import torch
    t0 = time.perf_counter()
    j = 0
    while j < count or time.perf_counter() - t0 < seconds:
        fn(j)
        j += 1
        if j % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return j


class Flush:
    """Evicts the L2 caches and the 256 MB last-level cache between cold
    iterations: a 1 GiB device write (torch's fill kernel), outside the
    timed interval."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.k = 0

    def __call__(self):
        self.k += 1
        self.buf.fill_(self.k & 0xFF)


def cold_steps(forward, n, flush):
    """n iterations of (flush; event; forward(j); event): per-step ms."""
    import torch
    out = []
    for j in range(n):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        forward(j)
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def build(wl, fp8):
    """Device inputs of one workload (resident in HBM) and the calls that
    make up its step."""
    import numpy as np
    import torch

    import hashed_head_gram_amd as pg
    import synth
    from synth import configs, device as sdev

    dev = torch.device("cuda:0")
    lay_d = wl["layout"]
    layout = pg.make_layout(lay_d["kind"], lay_d["K"], lay_d["r"], S=lay_d["S"],
                            pages=lay_d["pages"], head_rows=lay_d["head_rows"],
                            hash_seed=lay_d["hash_seed"], use_signs=lay_d["use_signs"],
                            n_min=lay_d["n_min"], n_max=lay_d["n_max"],
                            pad_id=wl["canon_vocab"])
    R = pg.pg_layout_rows(layout)
    r = lay_d["r"]
    B, T = wl["B"], wl["T"]
    N = B * T
    costs = algorithmic_costs(wl, fp8)
    E = costs["E"]
    if fp8 and (wl["act_dtype"] != "bf16" or E % 128):
        sys.exit(f"--fp8 needs bf16 activations and an e dimension that is a multiple of "
                 f"128 ({wl['name']}: {wl['act_dtype']}, {E})")
    act = torch.float32 if wl["act_dtype"] == "f32" else torch.bfloat16
    e_dtype = pg.PG_F32 if wl["act_dtype"] == "f32" else pg.PG_BF16
    keep = {}
    if wl["table_dtype"] == "nf4":
        codes = torch.empty(R, r // 2, dtype=torch.uint8, device=dev)
        scales = torch.empty(R, dtype=torch.float16, device=dev)
        sdev.fill_nf4_table(codes, scales, wl["table_seed"])
        table = pg.make_table(pg.PG_NF4, codes, R, scales=scales)
    else:
        tdt = torch.float32 if wl["table_dtype"] == "f32" else torch.bfloat16
        tab = torch.empty(R, r, dtype=tdt, device=dev)
        sdev.fill_normal(tab, wl["table_seed"], configs.STREAM_TABLE, wl["table_sigma"])
        table = pg.make_table(pg.PG_F32 if wl["table_dtype"] == "f32" else pg.PG_BF16,
                              tab, R)
    cmap = torch.from_numpy(synth.canon_map(wl)).to(dev)
    pool = [torch.from_numpy(synth.tokens(wl, batch=j)).to(dev) for j in range(POOL)]
    d_out = configs.d_out(wl)
    W = torch.empty(d_out, E, dtype=act, device=dev)
    sdev.fill_normal(W, wl["data_seed"], configs.STREAM_W, wl["w_sigma"])
    engram = wl["gate"] == "engram"
    if engram:
        M = wl["M"]
        gh, gk, gu, cw = (torch.from_numpy(np.ascontiguousarray(a)).to(dev)
                          for a in synth.engram_params(wl))
        fuse = pg.make_fuse(pg.PG_GATE_ENGRAM, e_dtype, wl["d"], M=M, eps=wl["eps"],
                            gamma_h=gh, gamma_k=gk, gamma_u=gu, conv_w=cw,
                            conv_k=wl["conv_k"], conv_dil=wl["conv_dil"])
        resid = torch.empty(M * N, wl["d"], dtype=act, device=dev)
        out = torch.empty(M * N, wl["d"], dtype=act, device=dev)
    else:
        fuse = pg.make_fuse(pg.PG_GATE_SCALAR, e_dtype, wl["d"], g=wl["g"])
        resid = torch.empty(N, wl["d"], dtype=act, device=dev)
        out = torch.empty(N, wl["d"], dtype=act, device=dev)
    sdev.fill_normal(resid, wl["data_seed"], configs.STREAM_RESID, wl["resid_sigma"])
    ws = torch.empty(pg.pg_workspace_size(layout, fuse, B, T), dtype=torch.uint8, device=dev)
    e = torch.empty(N, E, dtype=torch.uint8 if fp8 else act, device=dev)
    ws2 = torch.empty(max(pg.pg_workspace_size(None, fuse, B, T), 256), dtype=torch.uint8,
                      device=dev)
    keep.update(table=table, cmap=cmap, pool=pool, W=W, fuse=fuse, resid=resid, out=out,
                ws=ws, e=e, ws2=ws2)
    calls = {}
    if fp8:
        se = FP8_E_SCALE[wl["table_dtype"]]
        sw = FP8_W_SCALE
        W8 = torch.empty(d_out, E, dtype=torch.uint8, device=dev)
        pg.pg_quantize_fp8(W, pg.PG_BF16, sw, W8)
        keep["W8"] = W8

        def forward(j):
            pg.pg_forward_fp8(layout, table, fuse, pool[j % POOL], cmap, W8, se, sw, resid,
                              out, ws)

        calls["gather"] = lambda j: pg.pg_index_gather_fp8(layout, table, pool[j % POOL],
                                                           cmap, se, e)
        if engram:
            calls["pass1"] = lambda j: pg.pg_engram_project_fp8(fuse, e, B, T, W8, se, sw,
                                                                resid, ws2)
        else:
            calls["projection"] = lambda j: pg.pg_project_gate_fp8(fuse, e, B, T, W8, se, sw,
                                                                   resid, out, ws2)
    else:
        def forward(j):
            pg.pg_forward(layout, table, fuse, pool[j % POOL], cmap, W, resid, out, ws)

        calls["gather"] = lambda j: pg.pg_index_gather(layout, table, pool[j % POOL], cmap,
                                                       e_dtype, e)
        if engram:
            calls["pass1"] = lambda j: pg.pg_engram_project(fuse, e, B, T, W, resid, ws2)
        else:
            calls["projection"] = lambda j: pg.pg_project_gate(fuse, e, B, T, W, resid, out,
                                                               ws2)
    if engram:
        calls["gate"] = lambda j: pg.pg_engram_gate(fuse, B, T, ws2)
        calls["pass2"] = lambda j: pg.pg_engram_mix(fuse, B, T, resid, out, ws2)
    # pg_forward runs as pg_index_records -> pg_project_gathered (E gathered
    # inside the matrix kernel) for bf16 tables of 64-element rows under the
    # scalar gate; otherwise as pg_index_gather -> pg_project_gate.
    gathered = (not fp8 and wl["table_dtype"] == "bf16" and r == 64 and not engram)
    if gathered:
        rec = torch.empty(pg.records_bytes(layout, N), dtype=torch.uint8, device=dev)
        keep["rec"] = rec
        calls["records"] = lambda j: pg.pg_index_records(layout, pool[j % POOL], cmap, rec)
        calls["gathered"] = lambda j: pg.pg_project_gathered(layout, table, fuse, rec, B, T,
                                                             W, resid, out)
    return dict(wl=wl, N=N, R=R, E=E, costs=costs, fp8=fp8, engram=engram,
                gathered=gathered, forward=forward, calls=calls, out=out, keep=keep,
                layout=layout)


def check_compositions(b):
    """pg_forward equals its stage calls bit for bit: the two-kernel path
    (and the gathered pair where pg_forward takes it)."""
    import torch
    out, c = b["out"], b["calls"]
    b["forward"](0)
    ref = out.clone()

    def same():
        torch.cuda.synchronize()
        return bool(torch.equal(out.view(torch.uint8), ref.view(torch.uint8)))
    two = ["gather", "pass1", "gate", "pass2"] if b["engram"] else ["gather", "projection"]
    for k in two:
        c[k](0)
    res = {"forward_matches_two_stage": same()}
    if b["gathered"]:
        c["records"](0)
        c["gathered"](0)
        res["forward_matches_gathered_pair"] = same()
    del ref
    return res


def run_workload(name, args, primary):
    """Timed figures of one workload: the whole step and each kernel."""
    import torch

    from synth import configs

    wl = configs.workload(name)
    b = build(wl, args.fp8)
    N, costs, calls = b["N"], b["costs"], b["calls"]
    eq = check_compositions(b)
    steps = args.steps if primary else min(args.steps, SECONDARY_STEPS)
    nwarm = warm(b["forward"], args.warmup, WARM_S if primary else WARM_S_SECONDARY)

    # Timed region: K whole steps (pg_forward) back to back, a HIP event
    # before each step, synchronised on both sides.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(steps):
        ev[j].record()
        b["forward"](j)
    ev[steps].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_spread = spread([ev[j].elapsed_time(ev[j + 1]) for j in range(steps)])
    step_spread["mean"] = ev[0].elapsed_time(ev[steps]) / steps

    # Per-kernel launch durations: K launches of each stage call alone.
    kern = {k: per_launch(fn, steps) for k, fn in calls.items() if k != "records"}
    if b["gathered"]:
        kern["records"] = {"mean": records_graph_ms(calls["records"], b["keep"]["rec"], steps)}
    cold = None
    if primary and not args.no_cold:
        flush = Flush(torch.device("cuda:0"))
        cold = spread(cold_steps(b["forward"], min(steps, COLD_STEPS), flush))
        del flush

    ms_per_step = wall / steps * 1e3
    tkey = wl["name"] + ("/fp8" if args.fp8 else "")
    fp8 = args.fp8
    p_peak = (FP8_PEAK_TFLOPS if fp8 else
              FP32_PEAK_TFLOPS if wl["act_dtype"] == "f32" else BF16_PEAK_TFLOPS)
    g_bytes = costs["gather_bytes"] * N
    g = kern["gather"]
    gather_rec = {"kernel": "index_gather_kernel", "ms": g, "bytes_per_launch": g_bytes,
                  "achieved_GBps": g_bytes / (g["mean"] / 1e3) / 1e9,
                  "frac_hbm_peak": g_bytes / (g["mean"] / 1e3) / 1e9 / HBM_PEAK_GBPS,
                  "traffic": traffic_for("gather", tkey)}
    rec = {"workload": wl["name"], "tokens_per_step": N, "value": N / (ms_per_step / 1e3) / 1e6,
           "ms_per_step": ms_per_step, "step_ms_gpu_events": step_spread,
           "warmup_steps_run": nwarm, "gather": gather_rec}
    rec.update(eq)
    p_flops = costs["proj_flops"] * N
    if b["engram"]:
        p1 = kern["pass1"]
        tf = p_flops / (p1["mean"] / 1e3) / 1e12
        p1_bytes = costs["pass1_bytes"] * N
        p1_kernel = "engram_slot_kernel"
        rec["pass1"] = {"kernel": p1_kernel + " (Engram pass 1: [W_V; W_K] GEMM + "
                                  "partial-sum epilogue)", "ms": p1,
                        "flops_per_launch": p_flops, "achieved_TFLOPs": tf,
                        "frac_mfma_peak": tf / p_peak, "bytes_per_launch": p1_bytes,
                        "achieved_GBps": p1_bytes / (p1["mean"] / 1e3) / 1e9,
                        "traffic": traffic_for("pass1", tkey)}
        p2 = kern["pass2"]
        p2_bytes = costs["pass2_bytes"] * N
        rec["pass2"] = {"kernel": "engram_pass2_kernel", "ms": p2,
                        "bytes_per_launch": p2_bytes,
                        "achieved_GBps": p2_bytes / (p2["mean"] / 1e3) / 1e9,
                        "frac_hbm_peak": p2_bytes / (p2["mean"] / 1e3) / 1e9 / HBM_PEAK_GBPS,
                        "traffic": traffic_for("pass2", tkey)}
        rec["gate"] = {"kernel": "engram_gate_kernel", "ms": kern["gate"]}
        roof = {"kernel": p1_kernel, "bound": "mfma", "achieved": tf,
                "peak": p_peak, "unit": "TFLOP/s", "frac": tf / p_peak,
                "traffic": rec["pass1"]["traffic"]}
    else:
        pj = kern["projection"]
        tf = p_flops / (pj["mean"] / 1e3) / 1e12
        p_bytes = costs["proj_bytes"] * N
        rec["projection"] = {
            "kernel": ("gemm_pipe_kernel" if b["E"] % (128 if fp8 else 64) == 0
                       else "gemm_bf16_kernel") if wl["act_dtype"] == "bf16"
            else "gemm_f32_kernel",
            "ms": pj, "flops_per_launch": p_flops, "achieved_TFLOPs": tf,
            "frac_mfma_peak": tf / p_peak, "bytes_per_launch": p_bytes,
            "achieved_GBps": p_bytes / (pj["mean"] / 1e3) / 1e9,
            "traffic": traffic_for("projection", tkey)}
        roof = {"kernel": rec["projection"]["kernel"], "bound": "mfma", "achieved": tf,
                "peak": p_peak, "unit": "TFLOP/s", "frac": tf / p_peak,
                "traffic": rec["projection"]["traffic"]}
        if b["gathered"]:
            gp = kern["gathered"]
            OK = b["E"] // wl["layout"]["r"]
            gp_bytes = (costs["proj_bytes"] - b["E"] * 2 + OK * (2 * wl["layout"]["r"] + 16)) * N
            gtf = p_flops / (gp["mean"] / 1e3) / 1e12
            rec["gathered_projection"] = {
                "kernel": "gemm_pipe_gather_kernel", "ms": gp, "flops_per_launch": p_flops,
                "achieved_TFLOPs": gtf, "frac_mfma_peak": gtf / p_peak,
                "bytes_per_launch": gp_bytes,
                "achieved_GBps": gp_bytes / (gp["mean"] / 1e3) / 1e9,
                "traffic": traffic_for("gathered", tkey),
                "records_kernel_ms": kern["records"]["mean"],
                "records_bytes_per_launch": N * (4 + 16 * OK)}
            roof = {"kernel": "gemm_pipe_gather_kernel", "bound": "mfma", "achieved": gtf,
                    "peak": p_peak, "unit": "TFLOP/s", "frac": gtf / p_peak,
                    "traffic": rec["gathered_projection"]["traffic"]}
        elif g["mean"] > pj["mean"]:
            roof = {"kernel": "index_gather_kernel", "bound": "hbm",
                    "achieved": gather_rec["achieved_GBps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": gather_rec["frac_hbm_peak"],
                    "traffic": gather_rec["traffic"]}
    rec["roofline"] = roof
    if cold is not None:
        rec["cold_step_ms"] = cold
        rec["cold_value"] = N / (cold["median"] / 1e3) / 1e6
    rec["config"] = {"workload": wl["name"], "tokens_per_step": N, "batch": wl["B"],
                     "seq_len": wl["T"], "layout": wl["layout"]["kind"], "K": wl["layout"]["K"],
                     "S": wl["layout"]["S"], "r": wl["layout"]["r"],
                     "table_dtype": wl["table_dtype"], "table_rows": b["R"], "d": wl["d"],
                     "gate": wl["gate"], "token_pool": POOL}
    if b["engram"]:
        rec["config"]["M"] = wl["M"]
        rec["config"]["d_out"] = (1 + wl["M"]) * wl["d"]
    del b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def read_peak():
    """Streaming-read rate of this GPU (GB/s): the library's read probe over
    a 4 GiB buffer, median of 20 launches."""
    import torch

    import hashed_head_gram_amd as pg
    dev = torch.device("cuda:0")
    buf = torch.ones(READ_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    for _ in range(3):
        pg.pg_read_probe(buf, sink)
    t = per_launch(lambda j: pg.pg_read_probe(buf, sink), 20)
    del buf
    torch.cuda.empty_cache()
    return {"GBps": READ_PROBE_BYTES / (t["median"] / 1e3) / 1e9, "bytes": READ_PROBE_BYTES,
            "ms": t}


def main():
    args = parse()
    if args.traffic_from:
        if len(args.traffic_from) not in (2, 3):
            sys.exit("--traffic-from takes FETCH_CSV WRITE_CSV [RDREQ_CSV]")
        write_traffic(args.workload, *args.traffic_from)
        return
    if args.backward:
        print(json.dumps(backward_bench(args)), flush=True)
        return
    if args.host_table:
        print(json.dumps(host_table_bench(args)), flush=True)
        return
    if args.page_cache:
        line = {"metric": "flash reads per token under an LRU RAM page cache (4 KiB blocks)",
                "unit": "reads/token", "higher_is_better": False, "n_gpus": 1,
                "data": "synthetic (seeded Zipf token stream of the 20B workloads, "
                        f"{args.steps} batches of 16 x 4096 tokens)",
                "config": {"workload": "20B NF4 table, three layouts",
                           "cache_MiB": PAGE_CACHE_MIB},
                "layouts": page_cache(args.steps)}
        print(json.dumps(line), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from synth import configs

    main_rec = run_workload(args.workload, args, primary=True)
    others = {}
    if not args.only:
        for name in SECONDARY:
            if name != args.workload:
                others[name] = run_workload(name, args, primary=False)
    peak = read_peak() if not args.fp8 else None
    if copy_probe_needed(args):
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        bb = torch.empty_like(a)
        for _ in range(COPY_REPS):
            bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb
    cpu = None
    if not args.no_cpu_baseline and not args.fp8:
        cpu = cpu_baseline(configs.workload(args.workload), args.cpu_tokens)
    wl = configs.workload(args.workload)
    line = {
        "metric": "M tokens/s for hash+gather+project; gather HBM GB/s and % of peak"
                  + (" (FP8 E4M3 projection operands)" if args.fp8 else ""),
        "value": main_rec["value"], "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_rec["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 operands, fp32 accumulate, bf16 out" if args.fp8 else wl["act_dtype"],
        "data": "synthetic (seeded Zipf token streams, counter-generated table and weights)",
        "config": main_rec.pop("config"),
        "roofline": main_rec.pop("roofline"),
    }
    if peak is not None:
        line["measured_read_peak"] = peak
        g = main_rec["gather"]
        g["frac_measured_read_peak"] = g["achieved_GBps"] / peak["GBps"]
        if "pass2" in main_rec:
            main_rec["pass2"]["frac_measured_read_peak"] = (main_rec["pass2"]["achieved_GBps"]
                                                            / peak["GBps"])
    for k in ("value", "ms_per_step"):
        main_rec.pop(k)
    line.update(main_rec)
    line["other_workloads"] = others
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def copy_probe_needed(args):
    return args.copy_probe


if __name__ == "__main__":
    main()
