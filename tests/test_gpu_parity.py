"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integers (canonical IDs, hashes, rows, pages, sign words) and the gathered e
(fp32 / bf16 bit patterns) must match bit for bit. Outputs must be within
1e-5 (fp32 workload) or 2e-2 (bf16 / NF4 workloads) of the float64 oracle,
measured as max_i |got_i - want_i| / max(|want_i|, rms(want)).

The seven workloads run at their full sizes: every token is compared for the
index and for e on all of them, and for the output on the small ones; the
big ones compare the output on sampled positions (sequence starts, the
conv's left edge, sequence ends and 8,192 random positions, or 192 for the
27B fusion, whose oracle recomputes each position's conv window).
"""
import numpy as np
import pytest
import torch

import hashed_head_gram_amd as pg
import oracle
import synth
from synth import configs
from tests.gpu_inputs import Case, bf16_to_np, rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
_cases = {}


def case(i):
    if i not in _cases:
        print(f"[case] building workload {configs.ORDER[i]}", flush=True)
        _cases[i] = Case(configs.workload(i))
        torch.cuda.synchronize()
    return _cases[i]


def teardown_module(module):
    _cases.clear()
    torch.cuda.empty_cache()


def sample_positions(c, n_random=48, seed=0):
    rng = np.random.default_rng(seed)
    T = c.T
    pos = set()
    for b in sorted({0, c.B // 2, c.B - 1}):
        for t in (0, 1, 2, 3, 8, 9, 10, T - 2, T - 1):
            if 0 <= t < T:
                pos.add(b * T + t)
    pos |= set(rng.integers(0, c.N, size=n_random).tolist())
    return np.array(sorted(pos), dtype=np.int64)


def assert_bits_equal(got, want, what, row_len=None):
    """Bitwise equality with a report of where the arrays differ."""
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if len(bad):
        cols = bad[:, -1]
        msg = (f"{what}: {len(bad)} of {got.size} differ; first at {bad[:5].tolist()} "
               f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")
        if row_len:
            hist = np.bincount((cols % row_len) // 32, minlength=row_len // 32)
            msg += f"; by 32-element chunk of a row: {hist.tolist()}"
            msg += f"; rows affected: {np.unique(bad[:, 0]).size}"
        raise AssertionError(msg)


def full(c):
    return c.N <= 16384 and c.wl["gate"] == "scalar"


def e_as_np(c, e):
    if c.act == torch.float32:
        return e.cpu().numpy()
    return e.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("i", range(len(configs.ORDER)))
def test_index_bit_exact(i):
    c = case(i)
    got = c.run_index()
    torch.cuda.synchronize()
    ref = oracle.index(c.lay_d, c.tokens_np, c.cmap_np, c.pad)
    assert np.array_equal(got["canon"].cpu().numpy(), ref["canon"].reshape(-1))
    assert np.array_equal(got["hashes"].cpu().numpy().view(np.uint64), ref["hashes"])
    assert np.array_equal(got["rows"].cpu().numpy(), ref["rows"])
    assert np.array_equal(got["pages"].cpu().numpy(), ref["pages"])
    assert np.array_equal(got["signs"].cpu().numpy().view(np.uint64), ref["signs"])
    assert got["status"].item() == 0


@pytest.mark.parametrize("i", range(len(configs.ORDER)))
def test_gather_bit_exact(i):
    c = case(i)
    e = c.run_index_gather()
    idx = c.run_index()
    e2 = c.e_buffer()
    pg.pg_gather(c.layout, c.table, idx["rows"], idx["signs"], c.e_dtype, e2)
    torch.cuda.synchronize()
    # the fused kernel and index -> gather agree bit for bit
    assert torch.equal(e.view(torch.uint8), e2.view(torch.uint8))
    # every token against the oracle, in chunks (the big tables' rows are
    # regenerated on the host from the seeded generator, row by row)
    ref_idx = oracle.index(c.lay_d, c.tokens_np, c.cmap_np, c.pad)
    chunk = 16384
    for lo in range(0, c.N, chunk):
        pos = np.arange(lo, min(lo + chunk, c.N))
        want = oracle.gather_stored(c.lay_d, c.wl["table_dtype"], c.fetch,
                                    ref_idx["rows"][pos], ref_idx["signs"][pos])
        got = e_as_np(c, e[lo:lo + len(pos)])
        assert_bits_equal(got, want, f"e tokens {lo}..{lo + len(pos) - 1}", row_len=c.r)
        if c.N > chunk:
            print(f"[{configs.ORDER[i]}] e bit-exact through token {lo + len(pos)}", flush=True)


@pytest.mark.parametrize("i", range(len(configs.ORDER)))
def test_forward_within_tolerance(i):
    c = case(i)
    out = c.run_forward()
    inc = c.run_forward(increment_only=1)
    torch.cuda.synchronize()
    tol = TOL[c.wl["act_dtype"]]
    if c.wl["gate"] == "scalar":
        pos = np.arange(c.N) if full(c) else sample_positions(c, n_random=8192)
        ref = c.oracle_scalar(pos)
        ref_inc = c.oracle_scalar(pos, with_resid=False)
        sel = torch.from_numpy(pos).to(c.dev)
        got = out[sel].double().cpu().numpy()
        got_inc = inc[sel].double().cpu().numpy()
        err, err_inc = rel_err(got, ref["out"]), rel_err(got_inc, ref_inc["out"])
    else:
        pos = sample_positions(c, n_random=192)
        ref = c.oracle_engram(pos)
        ref_inc = c.oracle_engram(pos, with_resid=False)
        got = np.stack([out[m * c.N + torch.from_numpy(pos).to(c.dev)].double().cpu().numpy()
                        for m in range(c.M)])
        got_inc = np.stack([inc[m * c.N + torch.from_numpy(pos).to(c.dev)].double().cpu().numpy()
                            for m in range(c.M)])
        err, err_inc = rel_err(got, ref["out"]), rel_err(got_inc, ref_inc["out"])
    print(f"[{configs.ORDER[i]}] rel err out {err:.3e} increment {err_inc:.3e}")
    assert err < tol and err_inc < tol


@pytest.mark.parametrize("i", range(len(configs.ORDER)))
def test_forward_equals_stage_composition(i):
    # pg_forward == pg_index_gather -> pg_project_gate == pg_index -> pg_gather
    # -> pg_project_gate, bit for bit (same products, same summation order).
    c = case(i)
    out = c.run_forward()
    e = c.run_index_gather()
    out2 = c.run_project(e)
    idx = c.run_index()
    e3 = c.e_buffer()
    pg.pg_gather(c.layout, c.table, idx["rows"], idx["signs"], c.e_dtype, e3)
    out3 = c.run_project(e3)
    again = c.run_forward()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))
    assert torch.equal(out.view(torch.uint8), out3.view(torch.uint8))
    # run-to-run determinism
    assert torch.equal(out.view(torch.uint8), again.view(torch.uint8))


# ---------------------------------------------------------------------------
# Edge cases on small, ragged shapes (full element-wise comparison)


def small_wl(base, **kw):
    wl = configs.workload(base)
    lay = dict(wl["layout"])
    for k in ("kind", "K", "S", "r", "pages", "head_rows", "use_signs", "n_min", "n_max"):
        if k in kw:
            lay[k] = kw.pop(k)
    wl["layout"] = lay
    wl.update(kw)
    return wl


RAGGED = {
    "bf16_pagegram_B3_T37_d200": small_wl(1, pages=[97, 89], B=3, T=37, d=200),
    "bf16_engram_B2_T45_d256_r24": small_wl(4, K=4, r=24, head_rows=[101, 103, 107, 109,
                                                                      113, 127, 131, 137],
                                            B=2, T=45, d=256, M=2, gamma="random"),
    "f32_pagegram_K3_S5_r20_d50": small_wl(0, K=3, S=5, r=20, pages=[13, 11], B=2, T=33,
                                           d=50),
    "nf4_pagegram_r96_B2_T100": small_wl(3, r=96, pages=[31, 37], B=2, T=100, d=128),
    "nf4_pagegram_r96_B2_T96": small_wl(3, r=96, pages=[31, 37], B=2, T=96, d=128),
    "nf4_pagegram_r32_B2_T100": small_wl(3, r=32, pages=[31, 37], B=2, T=100, d=128),
    "nf4_pagegram_r64_B2_T100": small_wl(3, r=64, pages=[31, 37], B=2, T=100, d=128),
    "bf16_orders_1to4_K16": small_wl(1, K=16, S=2, r=16, n_min=1, n_max=4,
                                     pages=[5, 7, 11, 13], B=2, T=50, d=64),
    "bf16_nosigns_T1": small_wl(1, use_signs=0, pages=[7, 7], B=5, T=1, d=128),
    "bf16_engram_T2": small_wl(2, B=4, T=2, d=64),
    # e_dim 64: two 32-element K slots of the fused projection (the h tile's
    # first quarters are requested with the first slots); 600 tokens, d = 512,
    # three branches
    "bf16_engram_E64_two_slots": small_wl(4, K=2, r=16, head_rows=[101, 103, 107, 109], B=2,
                                          T=300, d=512, M=3, gamma="random"),
}


@pytest.mark.parametrize("name", list(RAGGED))
def test_ragged_cases_full_parity(name):
    wl = RAGGED[name]
    print(f"[ragged] {name}", flush=True)
    c = Case(wl)
    idx = c.run_index()
    e = c.run_index_gather()
    out = c.run_forward()
    torch.cuda.synchronize()
    ref = oracle.index(c.lay_d, c.tokens_np, c.cmap_np, c.pad)
    assert np.array_equal(idx["rows"].cpu().numpy(), ref["rows"])
    assert np.array_equal(idx["signs"].cpu().numpy().view(np.uint64), ref["signs"])
    assert np.array_equal(idx["hashes"].cpu().numpy().view(np.uint64), ref["hashes"])
    want_e = oracle.gather_stored(c.lay_d, wl["table_dtype"], c.fetch, ref["rows"],
                                  ref["signs"])
    e2 = c.e_buffer()
    pg.pg_gather(c.layout, c.table, idx["rows"], idx["signs"], c.e_dtype, e2)
    torch.cuda.synchronize()
    assert_bits_equal(e_as_np(c, e2), want_e, "pg_gather e", row_len=c.r)
    assert_bits_equal(e_as_np(c, e), want_e, "pg_index_gather e", row_len=c.r)
    pos = np.arange(c.N)
    tol = TOL[wl["act_dtype"]]
    if wl["gate"] == "scalar":
        r = c.oracle_scalar(pos)["out"]
        err = rel_err(out.double().cpu().numpy(), r)
    else:
        r = c.oracle_engram(pos)["out"]
        err = rel_err(out.double().cpu().numpy().reshape(c.M, c.N, c.d), r)
    print(f"[ragged] {name} rel err {err:.3e}")
    assert err < tol


def test_empty_inputs_enqueue_nothing():
    c = Case(small_wl(1, pages=[7, 7], B=2, T=8, d=64))
    out = torch.full((c.N, c.d), 3.0, dtype=torch.bfloat16, device=c.dev)
    e = torch.full((c.N, c.E), 5.0, dtype=torch.bfloat16, device=c.dev)
    f = c.fuse()
    empty = c.tokens[:0]
    pg.pg_index_gather(c.layout, c.table, empty, c.cmap, c.e_dtype, e)
    pg.pg_forward(c.layout, c.table, f, c.tokens[:, :0], c.cmap, c.W, c.resid, out, None)
    pg.pg_project_gate(f, e, 0, 8, c.W, c.resid, out)
    torch.cuda.synchronize()
    assert (out.float() == 3.0).all() and (e.float() == 5.0).all()


def test_out_of_range_tokens_map_to_pad_and_flag():
    wl = small_wl(1, pages=[11, 13], B=2, T=16, d=64)
    toks = synth.tokens(configs.with_tokens(wl, 2, 16))
    toks[0, 3] = -5
    toks[1, 7] = wl["vocab"] + 3
    c = Case(wl, tokens=toks)
    idx = c.run_index()
    st = torch.zeros(1, dtype=torch.int32, device=c.dev)
    c.run_index_gather(status=st)
    torch.cuda.synchronize()
    ref = oracle.index(c.lay_d, toks, c.cmap_np, c.pad)
    assert ref["bad"]
    assert idx["status"].item() == 1 and st.item() == 1
    assert np.array_equal(idx["canon"].cpu().numpy(), ref["canon"].reshape(-1))
    assert idx["canon"].cpu().numpy()[3] == c.pad
    assert np.array_equal(idx["rows"].cpu().numpy(), ref["rows"])


@pytest.mark.parametrize("base", [0, 1, 3, 4])
def test_zero_table_leaves_residual(base):
    # PageGram §9.4 check 3: a zero table reproduces the residual exactly
    # (compared by value: -0.0 and +0.0 are equal).
    if base == 4:
        wl = small_wl(4, K=8, r=80, head_rows=[53 + 2 * q for q in range(16)], B=2,
                      T=40, d=256, M=4)
    else:
        wl = configs.with_tokens(configs.workload(base), 2, 64)
        if base == 3:
            wl["layout"] = dict(wl["layout"], pages=[101, 103])
    c = Case(wl, zero_table=True)
    out = c.run_forward()
    torch.cuda.synchronize()
    assert torch.equal(out.float(), c.resid.float())


# The fused projection walks its tiles on one block per CU when E is a
# multiple of 128 (each tile's epilogue loads the next tile's first slots):
# about 1,000-1,600 tiles, so every block takes several, v and k tiles
# follow one another, and the ragged last M tile sits in the walk's last
# group, some of its k tiles with tiles after them. Outputs at tile edges,
# in the ragged tile and at random positions against the oracle.
TILE_WALK = {
    "E1280_d512_M3_N51000": dict(K=8, r=80, head_rows=[211 + 2 * q for q in range(16)], B=3,
                                 T=17000, d=512, M=3),
    "E128_d256_M3_N64006": dict(K=4, r=16, head_rows=[101, 103, 107, 109, 113, 127, 131, 137],
                                B=2, T=32003, d=256, M=3),
}


@pytest.mark.parametrize("name", list(TILE_WALK))
def test_engram_fusion_tile_walk(name):
    wl = small_wl(4, gamma="random", **TILE_WALK[name])
    print(f"[tile walk] {name}", flush=True)
    c = Case(wl)
    out = c.run_forward()
    torch.cuda.synchronize()
    pos = set(sample_positions(c, n_random=64).tolist())
    for t in range(0, c.N, 256 * 29):
        pos |= {t - 1, t, t + 255}
    pos |= set(range(c.N - 8, c.N))
    pos = np.array(sorted(q for q in pos if 0 <= q < c.N), dtype=np.int64)
    ref = c.oracle_engram(pos)
    sel = torch.from_numpy(pos).to(c.dev)
    got = np.stack([out[m * c.N + sel].double().cpu().numpy() for m in range(c.M)])
    err = rel_err(got, ref["out"])
    print(f"[tile walk] {name} rel err {err:.3e} over {len(pos)} positions")
    assert err < TOL[wl["act_dtype"]]
    # Every tile of the walk ran: with the workspace and the output filled
    # with NaN bytes beforehand, the stage calls leave no output NaN (a tile
    # left out would leave its v or partial sums NaN, and with them every
    # output that depends on them), and they equal pg_forward bit for bit.
    e = c.run_index_gather()
    f = c.fuse(0)
    ws = torch.full((max(pg.pg_workspace_size(None, f, c.B, c.T), 256),), 0xFF,
                    dtype=torch.uint8, device=c.dev)
    out2 = c.out_buffer()
    out2.view(torch.uint8).fill_(0xFF)
    pg.pg_engram_project(f, e, c.B, c.T, c.W, c.resid, ws)
    pg.pg_engram_gate(f, c.B, c.T, ws)
    pg.pg_engram_mix(f, c.B, c.T, c.resid, out2, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out2.float()).all())
    assert torch.equal(out2.view(torch.uint8), out.view(torch.uint8))


def test_causality_on_gpu():
    # Editing later tokens leaves earlier outputs bitwise unchanged, conv
    # included (Engram explainer, validation).
    wl = small_wl(4, K=8, r=80, head_rows=[211 + 2 * q for q in range(16)], B=2, T=64,
                  d=256, M=2)
    toks = synth.tokens(configs.with_tokens(wl, 2, 64))
    a = Case(wl, tokens=toks)
    out_a = a.run_forward().view(a.M, a.N, a.d)
    toks2 = toks.copy()
    toks2[:, 40:] = (toks2[:, 40:] * 7 + 3) % wl["vocab"]
    b = Case(wl, tokens=toks2)
    out_b = b.run_forward().view(b.M, b.N, b.d)
    torch.cuda.synchronize()
    keep = torch.from_numpy((np.arange(a.N) % 64) < 40).to(a.dev)
    assert torch.equal(out_a[:, keep].view(torch.int16), out_b[:, keep].view(torch.int16))
    assert not torch.equal(out_a[:, ~keep].view(torch.int16), out_b[:, ~keep].view(torch.int16))


def test_flat_special_case_bit_exact():
    # K=1, S=1, r=d with W = [I I]: the increment is g (s_2 T[h_2] + s_3 T[h_3])
    # exactly (PageGram §2.1); in fp32 each output is one rounding of a sum of
    # two table values, which the fp64 oracle rounded to fp32 reproduces.
    d = 64
    wl = small_wl(0, K=1, S=1, r=d, pages=[53, 59], B=2, T=50, d=d)
    c = Case(wl)
    eye = torch.eye(d, dtype=torch.float32, device=c.dev)
    c.W = torch.cat([eye, eye], dim=1).contiguous()
    c._W_np = np.concatenate([np.eye(d), np.eye(d)], axis=1).astype(np.float32)
    inc = c.run_forward(increment_only=1)
    torch.cuda.synchronize()
    want = c.oracle_scalar(np.arange(c.N), with_resid=False)["out"].astype(np.float32)
    assert np.array_equal(inc.cpu().numpy(), want)


def test_synth_device_fill_matches_host():
    # Every element, not a sample: rounding ties (fp32 -> fp16 scales,
    # fp32 -> bf16 values) must come out the same on both sides.
    from synth import device as sdev
    dev = torch.device("cuda:0")
    n = 1 << 20
    idx = np.arange(n)
    for dt, torch_dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        t = torch.empty(n, dtype=torch_dt, device=dev)
        sdev.fill_normal(t, 17, configs.STREAM_TABLE, 0.02, offset=5)
        host = synth.normal_values(17, configs.STREAM_TABLE, idx + 5, 0.02, dt)
        got = t.cpu().numpy() if dt == "f32" else t.view(torch.int16).cpu().numpy().view(np.uint16)
        assert_bits_equal(got, host, f"fill {dt}")
    wl = configs.workload(3)
    rows = 65536
    codes = torch.empty(rows, 32, dtype=torch.uint8, device=dev)
    scales = torch.empty(rows, dtype=torch.float16, device=dev)
    sdev.fill_nf4_table(codes, scales, wl["table_seed"])
    hc, hs = synth.table_rows(wl, np.arange(rows))
    assert_bits_equal(codes.cpu().numpy(), hc, "nf4 codes")
    assert_bits_equal(scales.cpu().numpy().view(np.uint16), hs.view(np.uint16), "nf4 scales")


@pytest.mark.parametrize("which", ["ragged", "full"])
def test_engram_stage_calls_equal_project_gate(which):
    # pg_project_gate with the Engram gate == pg_engram_project ->
    # pg_engram_gate -> pg_engram_mix, bit for bit (full and increment-only).
    c = case(4) if which == "full" else Case(RAGGED["bf16_engram_B2_T45_d256_r24"])
    e = c.run_index_gather()
    for inc in (0, 1):
        out = c.run_project(e, increment_only=inc)
        f = c.fuse(inc)
        ws = torch.empty(max(pg.pg_workspace_size(None, f, c.B, c.T), 256), dtype=torch.uint8,
                         device=c.dev)
        out2 = c.out_buffer()
        pg.pg_engram_project(f, e, c.B, c.T, c.W, c.resid, ws)
        pg.pg_engram_gate(f, c.B, c.T, ws)
        pg.pg_engram_mix(f, c.B, c.T, c.resid, out2, ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8)), (which, inc)
        del ws, out, out2
    with pytest.raises(pg.PagegramError):        # a scalar-gate fuse is refused
        fs = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, c.d)
        pg.pg_engram_gate(fs, c.B, c.T, torch.empty(256, dtype=torch.uint8, device=c.dev))
