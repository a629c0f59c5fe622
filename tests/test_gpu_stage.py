"""GPU parity of staging from a host-resident table (pg_stage_rows,
pg_gather_staged) against the oracle (oracle/stage.py) and the HBM path.

The source table is a pinned host copy of the device table. Bit-exact: e
gathered from the staged cache equals e gathered from the table; the
number of staged units and the set of their first rows equal the oracle's;
every cache slot holds its unit's rows.
"""
import numpy as np
import pytest
import torch

import hashed_head_gram_amd as pg
import oracle
from oracle import stage
from synth import configs
from tests.gpu_inputs import Case
from tests.test_gpu_parity import RAGGED, small_wl

pytestmark = pytest.mark.gpu

CASES = {
    "pagegram200m_bf16": configs.workload(1),
    "engram200m_bf16": configs.workload(2),
    "pagegram_nf4_ragged": RAGGED["nf4_pagegram_r64_B2_T100"],
    "engram_nf4_small": small_wl(6, head_rows=[1009, 1013, 1019, 1021, 1031, 1033, 1039, 1049,
                                               1051, 1061, 1063, 1069, 1087, 1091, 1093, 1097],
                                 B=2, T=300, d=256),
    "engram_bf16_r24_ragged": RAGGED["bf16_engram_B2_T45_d256_r24"],
    "tiny_fp32": configs.workload(0),
}

PG_DT = {"f32": pg.PG_F32, "bf16": pg.PG_BF16, "nf4": pg.PG_NF4}


def _host_table(c):
    """Pinned host copy of the device table, as a pg_table, plus its tensors."""
    if c.wl["table_dtype"] == "nf4":
        codes = torch.empty(c.codes.shape, dtype=torch.uint8, pin_memory=True)
        scales = torch.empty(c.scales.shape, dtype=torch.float16, pin_memory=True)
        codes.copy_(c.codes)
        scales.copy_(c.scales)
        return pg.make_table(pg.PG_NF4, codes, c.R, scales=scales), (codes, scales)
    tab = torch.empty(c.tab.shape, dtype=c.tab.dtype, pin_memory=True)
    tab.copy_(c.tab)
    return pg.make_table(PG_DT[c.wl["table_dtype"]], tab, c.R), (tab,)


def _cache(c, rows_cap):
    if c.wl["table_dtype"] == "nf4":
        codes = torch.zeros(rows_cap, c.r // 2, dtype=torch.uint8, device=c.dev)
        scales = torch.zeros(rows_cap, dtype=torch.float16, device=c.dev)
        return pg.make_table(pg.PG_NF4, codes, rows_cap, scales=scales), (codes, scales)
    tab = torch.zeros(rows_cap, c.r, dtype=c.tab.dtype, device=c.dev)
    return pg.make_table(PG_DT[c.wl["table_dtype"]], tab, rows_cap), (tab,)


def _as_bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


_cases = {}


def case(name):
    if name not in _cases:
        _cases.clear()
        c = Case(CASES[name])
        _cases[name] = (c, _host_table(c))
    return _cases[name]


def teardown_module(module):
    _cases.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["page", "row"])
@pytest.mark.parametrize("name", list(CASES))
def test_staged_gather_equals_table_gather(name, kind):
    wl = CASES[name]
    print(f"[stage] {name} {kind} units", flush=True)
    c, (src, host) = case(name)
    dt = PG_DT[wl["table_dtype"]]
    uk = pg.PG_STAGE_PAGE if kind == "page" else pg.PG_STAGE_ROW
    U, max_units, wsb = pg.pg_stage_geometry(c.layout, dt, c.N, unit_kind=uk)
    assert U == stage.unit_rows(c.lay_d, wl["table_dtype"], kind)
    cache, cache_t = _cache(c, max_units * U)
    idx = c.run_index()
    rows, signs = idx["rows"], idx["signs"]
    cache_rows = torch.full_like(rows, -1)
    n_units = torch.zeros(1, dtype=torch.int64, device=c.dev)
    unit_first = torch.full((max_units,), -1, dtype=torch.int64, device=c.dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=c.dev)
    pg.pg_stage_rows(c.layout, src, rows, cache, cache_rows, n_units, ws, unit_first=unit_first,
                     unit_kind=uk)
    e = c.e_buffer()
    pg.pg_gather_staged(c.layout, cache, cache_rows, signs, c.e_dtype, e)
    e_ref = c.run_index_gather()
    torch.cuda.synchronize()
    assert torch.equal(e.view(torch.uint8), e_ref.view(torch.uint8))
    # units against the oracle
    rows_np = rows.cpu().numpy()
    want_first, want_count = stage.staged_units(c.lay_d, wl["table_dtype"], rows_np, kind)
    n = int(n_units.item())
    assert n == len(want_first)
    got_first = unit_first[:n].cpu().numpy()
    assert np.array_equal(np.sort(got_first), want_first)
    # every slot holds its unit's rows; every lookup's cache row holds its row
    first_of = dict(zip(want_first.tolist(), want_count.tolist()))
    tab_b = _as_bytes(c.codes if dt == pg.PG_NF4 else c.tab).reshape(c.R, -1)
    cache_b = _as_bytes(cache_t[0]).reshape(max_units * U, -1)
    rng = np.random.default_rng(1)
    for s in sorted(set(rng.integers(0, n, size=min(n, 300)).tolist()) | {0, n - 1}):
        f = int(got_first[s])
        cnt = first_of[f]
        assert np.array_equal(cache_b[s * U:s * U + cnt], tab_b[f:f + cnt])
    cr = cache_rows.cpu().numpy()
    assert cr.min() >= 0 and cr.max() < max_units * U
    flat_r, flat_c = rows_np.reshape(-1), cr.reshape(-1)
    assert np.array_equal(cache_b[flat_c], tab_b[flat_r])
    if dt == pg.PG_NF4:
        assert np.array_equal(_as_bytes(cache_t[1]).reshape(-1, 2)[flat_c],
                              _as_bytes(c.scales).reshape(-1, 2)[flat_r])


def test_stage_rejects_small_cache_and_workspace():
    c = Case(small_wl(1, pages=[7, 5], B=2, T=8, d=64))
    src, host = _host_table(c)
    U, max_units, wsb = pg.pg_stage_geometry(c.layout, pg.PG_BF16, c.N)
    idx = c.run_index()
    cache, _ = _cache(c, max_units * U - 1)
    cr = torch.empty_like(idx["rows"])
    nu = torch.zeros(1, dtype=torch.int64, device=c.dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=c.dev)
    with pytest.raises(pg.PagegramError):
        pg.pg_stage_rows(c.layout, src, idx["rows"], cache, cr, nu, ws)
    cache, _ = _cache(c, max_units * U)
    with pytest.raises(pg.PagegramError):
        pg.pg_stage_rows(c.layout, src, idx["rows"], cache, cr, nu, ws[:wsb - 256])
