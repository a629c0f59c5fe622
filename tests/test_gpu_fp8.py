"""GPU parity of the FP8 (E4M3) operands and projection against the oracle
(oracle/fp8.py with the float64 path of oracle/pagegram.py).

Bit-exact: pg_quantize_fp8 on every bf16 bit pattern and on exact fp32
ties; the E4M3 e of pg_index_gather_fp8; pg_forward_fp8 against its two
stages. Within tolerance (fp32 accumulation, bf16 output): the projection
and the whole path against float64 products of the dequantised operands.

The oracle of the whole path quantises the table rows instead of e: E4M3
rounding is symmetric in sign, so quantising before or after the +-1 signs
gives the same codes, and every dequantised value is exact in bf16, so the
oracle reads a bf16 table of dequantised values.
"""
import numpy as np
import pytest
import torch

import hashed_head_gram_amd as pg
import oracle
from oracle import fp8
from synth import configs
from tests.gpu_inputs import Case, rel_err
from tests.test_gpu_parity import RAGGED, TILE_WALK, sample_positions, small_wl

pytestmark = pytest.mark.gpu

TOL = 1e-2            # fp32 accumulation + bf16 output rounding (2^-9)
TOL_ENGRAM = 2e-2     # the bf16 bound: the Engram chain also stores v in bf16
SE = {"bf16": 11, "f32": 11, "nf4": 13}   # e scale exponents (|e| 2^s well below 448)
SW = 10                                   # W ~ N(0, 0.05)


def _u8(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def _assert_bytes(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert not len(bad), (f"{what}: {len(bad)} of {got.size} bytes differ; first at "
                          f"{bad[:5].tolist()} got {got.reshape(-1)[bad[:5]].tolist()} "
                          f"want {want.reshape(-1)[bad[:5]].tolist()}")


def test_quantize_every_bf16_pattern():
    dev = torch.device("cuda:0")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    src = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    x = fp8.bf16_bits_to_f64(bits)
    for s in (0, 7, -3, 12):
        dst = torch.empty(65536, dtype=torch.uint8, device=dev)
        pg.pg_quantize_fp8(src, pg.PG_BF16, s, dst)
        torch.cuda.synchronize()
        _assert_bytes(dst.cpu().numpy(), fp8.quantize(x, s), f"bf16 patterns, s={s}")


def test_quantize_fp32_ties_and_ragged_length():
    dev = torch.device("cuda:0")
    v = fp8.e4m3_values()[:0x7F]
    mids = (v[:-1] + v[1:]) / 2                     # exact ties (<= 5 significant bits)
    rng = np.random.default_rng(9)
    x = np.concatenate([mids, -mids, v, rng.normal(0, 50, 4000), [1e30, -1e30, np.nan, -0.0]])
    x = x[: len(x) - (len(x) % 8) + 5]              # a tail shorter than 8 elements
    for s in (0, -4, 3):
        xs = (x * 2.0 ** -s).astype(np.float32)     # so that xs 2^s == x exactly
        src = torch.from_numpy(xs).to(dev)
        dst = torch.empty(len(xs), dtype=torch.uint8, device=dev)
        pg.pg_quantize_fp8(src, pg.PG_F32, s, dst)
        torch.cuda.synchronize()
        _assert_bytes(dst.cpu().numpy(), fp8.quantize(xs.astype(np.float64), s),
                      f"fp32 ties, s={s}")


def _stored_e_values(c, rows, signs):
    st = oracle.gather_stored(c.lay_d, c.wl["table_dtype"], c.fetch, rows, signs)
    if c.wl["table_dtype"] == "f32":
        return st.astype(np.float64)
    return fp8.bf16_bits_to_f64(st)


GATHER_CASES = {
    "pagegram200m_full": configs.workload(1),
    "tiny_fp32": configs.workload(0),
    "nf4_r96_ragged": RAGGED["nf4_pagegram_r96_B2_T100"],
    "engram_r24_ragged": RAGGED["bf16_engram_B2_T45_d256_r24"],
    "orders_1to4_K16": RAGGED["bf16_orders_1to4_K16"],
    "nosigns_T1": RAGGED["bf16_nosigns_T1"],
}


@pytest.mark.parametrize("name", list(GATHER_CASES))
def test_index_gather_fp8_bit_exact(name):
    print(f"[fp8 gather] {name}", flush=True)
    c = Case(GATHER_CASES[name])
    se = SE[c.wl["table_dtype"]]
    e8 = torch.empty(c.N, c.E, dtype=torch.uint8, device=c.dev)
    pg.pg_index_gather_fp8(c.layout, c.table, c.tokens, c.cmap, se, e8)
    torch.cuda.synchronize()
    ref = oracle.index(c.lay_d, c.tokens_np, c.cmap_np, c.pad)
    want = fp8.quantize(_stored_e_values(c, ref["rows"], ref["signs"]), se)
    _assert_bytes(e8.cpu().numpy(), want, f"{name} e8")


PROJ_SHAPES = [(300, 128, 200), (16384, 1024, 768), (1000, 1280, 512), (257, 256, 64)]


@pytest.mark.parametrize("N,E,d", PROJ_SHAPES)
def test_project_gate_fp8_scalar(N, E, d):
    print(f"[fp8 project] N={N} E={E} d={d}", flush=True)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(N + E + d)
    e8 = fp8.quantize(rng.normal(0, 0.02, (N, E)), 11)
    W8 = fp8.quantize(rng.normal(0, 0.05, (d, E)), SW)
    x = rng.normal(0, 1, (N, d)).astype(np.float32)
    xt = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    x64 = xt.double().cpu().numpy()
    g = 0.5
    y = fp8.project_fp8(e8, 11, W8, SW)
    for inc in (0, 1):
        f = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, d, g=g, increment_only=inc)
        out = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
        pg.pg_project_gate_fp8(f, _u8(e8, dev), 1, N, _u8(W8, dev), 11, SW, xt, out)
        torch.cuda.synchronize()
        want = g * y + (0 if inc else x64)
        err = rel_err(out.double().cpu().numpy(), want)
        print(f"[fp8 project] N={N} E={E} d={d} increment_only={inc} rel err {err:.3e}")
        assert err < TOL


class _Fp8Table:
    """Oracle accessors for the FP8 path: table rows replaced by their
    dequantised E4M3 values (as bf16 bit patterns), W by dequantised W8."""

    def __init__(self, c, se):
        self.c, self.se = c, se

    def fetch(self, rows):
        c = self.c
        st = c.fetch(np.asarray(rows, dtype=np.int64))
        dt = c.wl["table_dtype"]
        if dt == "bf16":
            v = fp8.bf16_bits_to_f64(st)
        elif dt == "f32":
            v = np.asarray(st, np.float32).astype(np.float64)
        else:                           # NF4: fp32(level * scale), then bf16, as stored in e
            codes, scales = st
            q = oracle.nf4_unpack(codes, c.r)
            prod = (oracle.nf4_codebook()[q] *
                    np.asarray(scales, np.float16).astype(np.float32)[:, None]).astype(np.float32)
            v = fp8.bf16_bits_to_f64(oracle.pagegram._f32_to_bf16_bits(prod))
        q = fp8.dequantize(fp8.quantize(v, self.se), self.se)
        return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _w8(c):
    W = c.W_np().astype(np.float64)
    W8 = fp8.quantize(W, SW)
    return W8, fp8.dequantize(W8, SW)


FWD_CASES = {
    "bf16_pagegram_ragged": RAGGED["bf16_pagegram_B3_T37_d200"],
    "nf4_r64_ragged": RAGGED["nf4_pagegram_r64_B2_T100"],
    "engram_r32_ragged": small_wl(4, K=4, r=32, head_rows=[101, 103, 107, 109, 113, 127, 131,
                                                           137], B=2, T=45, d=256, M=2,
                                  gamma="random"),
    # e_dim 128: two 64-element K slots, so the h tile's first quarters are
    # requested with the first slots; 600 tokens (a ragged third row tile),
    # d = 512, three branches
    "engram_E128_two_slots": small_wl(4, K=4, r=16, head_rows=[101, 103, 107, 109, 113, 127,
                                                               131, 137], B=2, T=300, d=512,
                                      M=3, gamma="random"),
}


@pytest.mark.parametrize("name", list(FWD_CASES))
def test_forward_fp8_vs_oracle_and_stages(name):
    wl = FWD_CASES[name]
    print(f"[fp8 forward] {name}", flush=True)
    c = Case(wl)
    se = SE[wl["table_dtype"]]
    W8, Wq = _w8(c)
    W8t = _u8(W8, c.dev)
    f = c.fuse()
    ws = torch.empty(max(pg.pg_workspace_size(c.layout, f, c.B, c.T), 256), dtype=torch.uint8,
                     device=c.dev)
    out = c.out_buffer()
    pg.pg_forward_fp8(c.layout, c.table, f, c.tokens, c.cmap, W8t, se, SW, c.resid, out, ws)
    # the two stages give the same bits
    e8 = torch.empty(c.N, c.E, dtype=torch.uint8, device=c.dev)
    pg.pg_index_gather_fp8(c.layout, c.table, c.tokens, c.cmap, se, e8)
    ws2 = torch.empty(max(pg.pg_workspace_size(None, f, c.B, c.T), 256), dtype=torch.uint8,
                      device=c.dev)
    out2 = c.out_buffer()
    pg.pg_project_gate_fp8(f, e8, c.B, c.T, W8t, se, SW, c.resid, out2, ws2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))
    # against the oracle on dequantised operands
    qt = _Fp8Table(c, se)
    pos = np.arange(c.N)
    if wl["gate"] == "scalar":
        ref = oracle.forward_scalar(c.lay_d, c.pad, c.tokens_np, c.cmap_np, "bf16", qt.fetch,
                                    Wq, wl["g"], lambda p: c.resid_rows(p), positions=pos)
        got = out.double().cpu().numpy()
    else:
        gh, gk, gu, cw = c.eng_np
        N = c.N
        ref = oracle.forward_engram(c.lay_d, c.pad, c.tokens_np, c.cmap_np, "bf16", qt.fetch,
                                    Wq, c.d, c.M, gh, gk, gu, cw, wl["conv_dil"], wl["eps"],
                                    lambda m, fl: c.resid_rows([m * N + fl])[0].astype(np.float64),
                                    positions=pos)
        got = out.double().cpu().numpy().reshape(c.M, c.N, c.d)
    err = rel_err(got, ref["out"])
    print(f"[fp8 forward] {name} rel err {err:.3e}")
    assert err < (TOL if wl["gate"] == "scalar" else TOL_ENGRAM)


def test_forward_fp8_tile_walk():
    # The E4M3 fused projection walks 1,600 tiles on one block per CU (20
    # slots of 64 elements), several per block, the last M tile ragged: every
    # output written (workspaces and outputs NaN-filled beforehand) and equal
    # between pg_forward_fp8 and its two stages; sampled positions, tile edges
    # and the ragged tile against the oracle on dequantised operands.
    wl = small_wl(4, gamma="random", **TILE_WALK["E1280_d512_M3_N51000"])
    print("[fp8 tile walk] E1280_d512_M3_N51000", flush=True)
    c = Case(wl)
    se = SE[wl["table_dtype"]]
    W8, Wq = _w8(c)
    W8t = _u8(W8, c.dev)
    f = c.fuse()

    def nan_bytes(n):
        return torch.full((max(n, 256),), 0xFF, dtype=torch.uint8, device=c.dev)

    ws = nan_bytes(pg.pg_workspace_size(c.layout, f, c.B, c.T))
    out = c.out_buffer()
    out.view(torch.uint8).fill_(0xFF)
    pg.pg_forward_fp8(c.layout, c.table, f, c.tokens, c.cmap, W8t, se, SW, c.resid, out, ws)
    e8 = torch.empty(c.N, c.E, dtype=torch.uint8, device=c.dev)
    pg.pg_index_gather_fp8(c.layout, c.table, c.tokens, c.cmap, se, e8)
    ws2 = nan_bytes(pg.pg_workspace_size(None, f, c.B, c.T))
    out2 = c.out_buffer()
    out2.view(torch.uint8).fill_(0xFF)
    pg.pg_project_gate_fp8(f, e8, c.B, c.T, W8t, se, SW, c.resid, out2, ws2)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))
    qt = _Fp8Table(c, se)
    pos = set(sample_positions(c, n_random=48).tolist())
    for t in range(0, c.N, 256 * 29):
        pos |= {t - 1, t, t + 255}
    pos |= set(range(c.N - 8, c.N))
    pos = np.array(sorted(q for q in pos if 0 <= q < c.N), dtype=np.int64)
    gh, gk, gu, cw = c.eng_np
    N = c.N
    ref = oracle.forward_engram(c.lay_d, c.pad, c.tokens_np, c.cmap_np, "bf16", qt.fetch, Wq,
                                c.d, c.M, gh, gk, gu, cw, wl["conv_dil"], wl["eps"],
                                lambda m, fl: c.resid_rows([m * N + fl])[0].astype(np.float64),
                                positions=pos)
    sel = torch.from_numpy(pos).to(c.dev)
    got = np.stack([out[m * c.N + sel].double().cpu().numpy() for m in range(c.M)])
    err = rel_err(got, ref["out"])
    print(f"[fp8 tile walk] rel err {err:.3e} over {len(pos)} positions")
    assert err < TOL_ENGRAM


def test_fp8_entry_points_reject_bad_arguments():
    c = Case(small_wl(1, pages=[7, 5], B=2, T=8, d=64))
    f = c.fuse()
    e8 = torch.zeros(c.N, c.E, dtype=torch.uint8, device=c.dev)
    W8 = torch.zeros(c.d, c.E, dtype=torch.uint8, device=c.dev)
    out = c.out_buffer()
    with pytest.raises(pg.PagegramError):          # scale exponent out of range
        pg.pg_project_gate_fp8(f, e8, c.B, c.T, W8, 65, 0, c.resid, out)
    with pytest.raises(pg.PagegramError):          # e_dim not a multiple of 128
        pg.pg_project_gate_fp8(f, e8[:, :64].contiguous(), c.B, c.T, W8[:, :64].contiguous(),
                               0, 0, c.resid, out)
    with pytest.raises(pg.PagegramError):
        pg.pg_quantize_fp8(c.W, pg.PG_NF4, 0, W8)


# ---------------------------------------------------------------------------
# FP8 at the full sizes of the 20B NF4 workload (scalar gate, 65,536 tokens,
# d = 2560) and of the 27B Engram fusion (131,072 tokens, the fused
# [W_V; W_K^(1..4)] GEMM of 12,800 x 1,280, gate and conv): sampled
# positions against the oracle on the dequantised operands.

_full = {}


def _full_case(i):
    if i not in _full:
        _full.clear()
        torch.cuda.empty_cache()
        print(f"[fp8 full] building workload {configs.ORDER[i]}", flush=True)
        _full[i] = Case(configs.workload(i))
        torch.cuda.synchronize()
    return _full[i]


def teardown_module(module):
    _full.clear()
    torch.cuda.empty_cache()


def _sample_positions(c, n_random, seed=0):
    rng = np.random.default_rng(seed)
    pos = set()
    for b in sorted({0, c.B // 2, c.B - 1}):
        for t in (0, 1, 2, 3, 8, 9, 10, c.T - 2, c.T - 1):
            pos.add(b * c.T + t)
    pos |= set(rng.integers(0, c.N, size=n_random).tolist())
    return np.array(sorted(pos), dtype=np.int64)


@pytest.mark.parametrize("i", [3, 4])
def test_forward_fp8_full_size(i):
    c = _full_case(i)
    wl = c.wl
    se = SE[wl["table_dtype"]]
    print(f"[fp8 full] {wl['name']} N={c.N} E={c.E} d={c.d}", flush=True)
    W8, Wq = _w8(c)
    W8t = _u8(W8, c.dev)
    f = c.fuse()
    ws = torch.empty(pg.pg_workspace_size(c.layout, f, c.B, c.T), dtype=torch.uint8,
                     device=c.dev)
    out = c.out_buffer()
    pg.pg_forward_fp8(c.layout, c.table, f, c.tokens, c.cmap, W8t, se, SW, c.resid, out, ws)
    torch.cuda.synchronize()
    del ws
    qt = _Fp8Table(c, se)
    if wl["gate"] == "scalar":
        pos = _sample_positions(c, 2000)
        ref = oracle.forward_scalar(c.lay_d, c.pad, c.tokens_np, c.cmap_np, "bf16", qt.fetch,
                                    Wq, wl["g"], lambda p: c.resid_rows(p), positions=pos)
        got = out[torch.from_numpy(pos).to(c.dev)].double().cpu().numpy()
        tol = TOL
    else:
        pos = _sample_positions(c, 24)
        gh, gk, gu, cw = c.eng_np
        N = c.N
        ref = oracle.forward_engram(c.lay_d, c.pad, c.tokens_np, c.cmap_np, "bf16", qt.fetch,
                                    Wq, c.d, c.M, gh, gk, gu, cw, wl["conv_dil"], wl["eps"],
                                    lambda m, fl: c.resid_rows([m * N + fl])[0].astype(np.float64),
                                    positions=pos)
        sel = torch.from_numpy(pos).to(c.dev)
        got = np.stack([out[m * N + sel].double().cpu().numpy() for m in range(c.M)])
        tol = TOL_ENGRAM
    err = rel_err(got, ref["out"])
    print(f"[fp8 full] {wl['name']} {len(pos)} positions rel err {err:.3e}", flush=True)
    assert err < tol
