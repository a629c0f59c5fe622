"""Throughput of the n-gram memory hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pg_forward call over one batch of synthetic tokens: canonical
map, n-grams, hashes, rows, gather/dequant/sign, concatenation, W_V
projection and fusion. Steps cycle through a pool of 32 distinct token
batches already resident in HBM, so the table rows of one step are not left
in the caches by the previous one.

The timed region is K steps back to back (wall clock and HIP events around
it). Each kernel's launch duration is then measured the same way, K launches
of that stage's entry point alone between HIP events on the stream it runs
on: pg_index_gather and pg_project_gate, the two calls pg_forward makes
(checked bit for bit once).

Prints one JSON line: whole-job tokens/s, the roofline position of the
dominant kernel (algorithmic bytes or flops per launch over its mean launch
duration), both kernels' figures, and the CPU oracle timed on a bounded
sample on the host cores.

--fp8 times the same path with E4M3 projection operands instead
(pg_forward_fp8 = pg_index_gather_fp8 + pg_project_gate_fp8; W quantised
once before timing): a separate line at another precision, never the
headline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector
POOL = 32
DEFAULT_WORKLOAD = "pagegram200m_bf16_8x2048"
# E4M3 scale exponents of the --fp8 mode: e ~ N(0, 0.02) rows (NF4: |e| <=
# about 0.05) and W ~ N(0, 0.05) times 2^s stay well below 448
FP8_E_SCALE = {"bf16": 11, "nf4": 13, "f32": 11}
FP8_W_SCALE = 10


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    # about 0.1 s of untimed steps: the GPU reaches its steady clocks before
    # the timed region (20 steps measure 10-15% slower)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=16384)
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
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write profiles/traffic.json from two rocprofv3 --pmc counter "
                        "collections (FETCH_SIZE, WRITE_SIZE) of a --copy-probe run")
    return p.parse_args()


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
    if wl["gate"] == "engram":
        M, d = wl["M"], wl["d"]
        flops = 2 * E * (1 + M) * d
        proj_bytes = E * e_elt + 2 * M * d * elt   # e in; h in, out (pass 1 + 2 read h)
    else:
        d = wl["d"]
        flops = 2 * E * d
        proj_bytes = E * e_elt + 2 * d * elt       # e in; x in, out
    return dict(gather_bytes=gather_bytes, proj_flops=flops, proj_bytes=proj_bytes, E=E)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gather": ["hashed_head_gram_amd/csrc/index.hip", "hashed_head_gram_amd/csrc/common.h"],
    "projection": ["hashed_head_gram_amd/csrc/gemm.hip", "hashed_head_gram_amd/csrc/common.h"],
    "gathered": ["hashed_head_gram_amd/csrc/gemm.hip", "hashed_head_gram_amd/csrc/common.h"],
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
TRAFFIC_KERNELS = {"gather": "index_gather_kernel", "projection": "gemm_pipe_kernel",
                   "gathered": "gemm_pipe_gather_kernel", "copy": "copyBuffer"}


def counter_means(path, counter):
    """Mean per-dispatch value (KiB) of one counter for each kernel family."""
    import csv
    sums = {}
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter:
            continue
        for fam, key in TRAFFIC_KERNELS.items():
            if key in row["Kernel_Name"]:
                d = sums.setdefault(fam, {})
                d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    # the copy family: only the 1 GiB probe copies (bench.py's other copies are
    # at most a third of that; FETCH_SIZE reads half of a copy's bytes)
    if "copy" in sums:
        sums["copy"] = {k: v for k, v in sums["copy"].items() if v * 1024 > 0.45 * COPY_BYTES}
    return {fam: sum(d.values()) / len(d) for fam, d in sums.items() if d}


def write_traffic(workload, fetch_csv, write_csv):
    """HBM bytes per launch of the gather and projection kernels (and of the
    gathered projection where the workload runs it): FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the
    1 GiB device copy read and write exactly 1 GiB."""
    fetch = counter_means(fetch_csv, "FETCH_SIZE")
    write = counter_means(write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / (fetch["copy"] * 1024)
    w_scale = COPY_BYTES / (write["copy"] * 1024)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    ent = {}
    for stage in ("gather", "projection", "gathered"):
        if stage not in fetch or stage not in write:
            continue
        rd = fetch[stage] * 1024 * f_scale
        wr = write[stage] * 1024 * w_scale
        ent[stage] = {"kernel": TRAFFIC_KERNELS[stage],
                      "source_digest": source_digest(KERNEL_SOURCES[stage]),
                      "fetch_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr,
                      "fetch_kib_raw": fetch[stage], "write_kib_raw": write[stage]}
    ent["copy_scale"] = {"fetch": f_scale, "write": w_scale,
                         "copy_fetch_kib_raw": fetch["copy"], "copy_write_kib_raw": write["copy"]}
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


def cpu_baseline(wl, n_tok, min_seconds=10.0, max_batches=64):
    """The CPU oracle on successive n_tok-token batches of the workload's
    stream (distinct seeded batches), until about min_seconds of timed work."""
    import numpy as np

    import oracle
    import synth
    from synth import configs

    T = wl["T"]
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
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {"value": batches * N / total / 1e6, "unit": "Mtok/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"{batches} batches of {B}x{Tn} tokens ({batches * N} tokens, the "
                      f"first batches of the seeded stream), {total:.1f} s timed; index and "
                      f"gather single-threaded numpy, fp64 GEMM on {blas} BLAS threads"}


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


def main():
    args = parse()
    if args.traffic_from:
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
    r = lay_d["r"]
    B, T = wl["B"], wl["T"]
    N = B * T
    fp8 = args.fp8
    costs = algorithmic_costs(wl, fp8)
    E = costs["E"]
    if fp8 and (wl["act_dtype"] != "bf16" or E % 128):
        sys.exit(f"--fp8 needs bf16 activations and an e dimension that is a multiple of "
                 f"128 ({wl['name']}: {wl['act_dtype']}, {E})")
    act = torch.float32 if wl["act_dtype"] == "f32" else torch.bfloat16
    e_dtype = pg.PG_F32 if wl["act_dtype"] == "f32" else pg.PG_BF16

    # Inputs, resident in HBM before timing.
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
    if wl["gate"] == "engram":
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
    # pg_forward's constituents, for per-kernel timing.
    e = torch.empty(N, E, dtype=torch.uint8 if fp8 else act, device=dev)
    ws2 = torch.empty_like(ws)
    if fp8:
        # E4M3 scale exponents: |e| 2^se and |W| 2^sw stay well below 448
        se = FP8_E_SCALE[wl["table_dtype"]]
        sw = FP8_W_SCALE
        W8 = torch.empty(d_out, E, dtype=torch.uint8, device=dev)
        pg.pg_quantize_fp8(W, pg.PG_BF16, sw, W8)

        def forward(j):
            pg.pg_forward_fp8(layout, table, fuse, pool[j % POOL], cmap, W8, se, sw, resid,
                              out, ws)

        def gather_call(j):
            pg.pg_index_gather_fp8(layout, table, pool[j % POOL], cmap, se, e)

        def project_call(j):
            pg.pg_project_gate_fp8(fuse, e, B, T, W8, se, sw, resid, out, ws2)
    else:
        def forward(j):
            pg.pg_forward(layout, table, fuse, pool[j % POOL], cmap, W, resid, out, ws)

        def gather_call(j):
            pg.pg_index_gather(layout, table, pool[j % POOL], cmap, e_dtype, e)

        def project_call(j):
            pg.pg_project_gate(fuse, e, B, T, W, resid, out, ws2)
    # pg_forward runs as pg_index_records -> pg_project_gathered (E gathered
    # inside the matrix kernel) for bf16 tables of 64-element rows under the
    # scalar gate; otherwise as pg_index_gather -> pg_project_gate.
    gathered = (not fp8 and wl["table_dtype"] == "bf16" and r == 64
                and wl["gate"] == "scalar")
    if gathered:
        rec = torch.empty(pg.records_bytes(layout, N), dtype=torch.uint8, device=dev)

        def records_call(j):
            pg.pg_index_records(layout, pool[j % POOL], cmap, rec)

        def gathered_call(j):
            pg.pg_project_gathered(layout, table, fuse, rec, B, T, W, resid, out)
    torch.cuda.synchronize()

    # The stage calls reproduce pg_forward bit for bit.
    out_fwd = torch.empty_like(out)
    forward(0)
    out_fwd.copy_(out)
    if gathered:
        records_call(0)
        gathered_call(0)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.uint8), out_fwd.view(torch.uint8))
    gather_call(0)
    project_call(0)
    torch.cuda.synchronize()
    same_two_stage = torch.equal(out.view(torch.uint8), out_fwd.view(torch.uint8))
    if not gathered:
        same = same_two_stage
    del out_fwd

    for j in range(args.warmup):
        forward(j)
    # Timed region: K whole steps (pg_forward) back to back.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for j in range(args.steps):
        forward(j)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_gpu_ms = ev0.elapsed_time(ev1) / args.steps

    # Per-kernel launch durations: K launches of each stage back to back
    # between HIP events on the stream they run on.
    def per_launch_ms(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for j in range(args.steps):
            fn(j)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps
    g_ms = np.array([per_launch_ms(gather_call)])
    p_ms = np.array([per_launch_ms(project_call)])
    gp_ms = np.array([per_launch_ms(gathered_call)]) if gathered else None
    rec_ms = records_graph_ms(records_call, rec, args.steps) if gathered else None

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()

    ms_per_step = wall / args.steps * 1e3
    tok_s = N / (ms_per_step / 1e3)
    g_bytes = costs["gather_bytes"] * N
    p_flops = costs["proj_flops"] * N
    p_bytes = costs["proj_bytes"] * N
    g_gbps = g_bytes / (g_ms.mean() / 1e3) / 1e9
    p_peak = (FP8_PEAK_TFLOPS if fp8 else
              FP32_PEAK_TFLOPS if wl["act_dtype"] == "f32" else BF16_PEAK_TFLOPS)
    tkey = wl["name"] + ("/fp8" if fp8 else "")
    p_tflops = p_flops / (p_ms.mean() / 1e3) / 1e12
    gather_rec = {"kernel": "index_gather_kernel", "ms_mean": float(g_ms.mean()),
                  "bytes_per_launch": g_bytes, "achieved_GBps": g_gbps,
                  "frac_hbm_peak": g_gbps / HBM_PEAK_GBPS,
                  "traffic": traffic_for("gather", tkey)}
    proj = {"kernel": ("gemm_pipe_kernel" if E % (128 if fp8 else 64) == 0 else "gemm_bf16_kernel")
            if act == torch.bfloat16 else "gemm_f32_kernel",
            "ms_mean": float(p_ms.mean()), "flops_per_launch": p_flops,
            "achieved_TFLOPs": p_tflops, "frac_mfma_peak": p_tflops / p_peak,
            "bytes_per_launch": p_bytes,
            "achieved_GBps": p_bytes / (p_ms.mean() / 1e3) / 1e9,
            "traffic": traffic_for("projection", tkey)}
    sfx = "_fp8" if fp8 else ""
    stages = {f"pg_index_gather{sfx}_ms": float(g_ms.mean()),
              f"pg_project_gate{sfx}_ms": float(p_ms.mean())}
    gathered_rec = None
    if gathered:
        # the matrix kernel reads each token's 2K table rows and records
        # (16 B per head slot) besides x and out
        OK = costs["E"] // r
        gp_bytes = (costs["proj_bytes"] - E * 2 + OK * (2 * r + 16)) * N
        gp_tflops = p_flops / (gp_ms.mean() / 1e3) / 1e12
        gathered_rec = {
            "kernel": "gemm_pipe_gather_kernel", "ms_mean": float(gp_ms.mean()),
            "flops_per_launch": p_flops, "achieved_TFLOPs": gp_tflops,
            "frac_mfma_peak": gp_tflops / p_peak, "bytes_per_launch": gp_bytes,
            "achieved_GBps": gp_bytes / (gp_ms.mean() / 1e3) / 1e9,
            "traffic": traffic_for("gathered", tkey),
            # records_kernel: the rest of a step (K launches of the pair take
            # step_ms_gpu_events each)
            "records_kernel_ms_derived": step_gpu_ms - float(gp_ms.mean()),
            # records_kernel alone: K launches captured in a HIP graph and
            # replayed (a launch costs the host more than this kernel takes)
            "records_kernel_ms": rec_ms,
            "records_bytes_per_launch": N * (4 + 16 * OK)}
        stages["pg_project_gathered_ms"] = float(gp_ms.mean())
        roof = {"kernel": gathered_rec["kernel"], "bound": "mfma", "achieved": gp_tflops,
                "peak": p_peak, "unit": "TFLOP/s", "frac": gp_tflops / p_peak,
                "traffic": gathered_rec["traffic"]}
    elif g_ms.mean() >= p_ms.mean():
        roof = {"kernel": gather_rec["kernel"], "bound": "hbm", "achieved": g_gbps,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": g_gbps / HBM_PEAK_GBPS,
                "traffic": gather_rec["traffic"]}
    else:
        roof = {"kernel": proj["kernel"], "bound": "mfma", "achieved": p_tflops,
                "peak": p_peak, "unit": "TFLOP/s", "frac": p_tflops / p_peak,
                "traffic": proj["traffic"]}
    cpu = None
    if not args.no_cpu_baseline and not fp8:
        cpu = cpu_baseline(wl, args.cpu_tokens)
    line = {
        "metric": "M tokens/s for hash+gather+project; gather HBM GB/s and % of peak"
                  + (" (FP8 E4M3 projection operands)" if fp8 else ""),
        "value": tok_s / 1e6, "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 operands, fp32 accumulate, bf16 out" if fp8 else wl["act_dtype"],
        "data": "synthetic (seeded Zipf token streams, counter-generated table and weights)",
        "config": {"workload": wl["name"], "tokens_per_step": N, "batch": B, "seq_len": T,
                   "layout": lay_d["kind"], "K": lay_d["K"], "S": lay_d["S"], "r": r,
                   "table_dtype": wl["table_dtype"], "table_rows": R, "d": wl["d"],
                   "gate": wl["gate"], "token_pool": POOL},
        "roofline": roof,
        "step_ms_gpu_events": step_gpu_ms,
        "stages": stages,
        "forward_path": ("pg_index_records -> pg_project_gathered" if gathered else
                         "pg_index_gather -> pg_project_gate"),
        "gathered_projection": gathered_rec,
        "gather": gather_rec,
        "projection": proj,
        "forward_matches_stage_calls": bool(same),
        "forward_matches_two_stage": bool(same_two_stage),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
