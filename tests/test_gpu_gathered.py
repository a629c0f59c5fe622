"""GPU parity of the gathered projection (pg_index_records ->
pg_project_gathered), the path pg_forward takes for bf16 tables of 64-element
rows under the scalar gate.

Bit-exact: every record decodes to pg_index's row and sign word (and those
equal the oracle's), and the projection equals pg_index_gather followed by
pg_project_gate bit for bit (same products, same summation order), with and
without the residual, over ragged token counts and output widths that take
both tile shapes and the edge tiles.
"""
import numpy as np
import pytest
import torch

import hashed_head_gram_amd as pg
import oracle
import synth
from synth import configs
from tests.gpu_inputs import Case, rel_err
from tests.test_gpu_parity import small_wl

pytestmark = pytest.mark.gpu

CASES = {
    "pagegram200m_bf16": configs.workload(1),
    "engram200m_bf16": configs.workload(2),
    "pagegram_B3_T37_d200": small_wl(1, pages=[97, 89], B=3, T=37, d=200),
    "pagegram_B2_T300_d256": small_wl(1, pages=[97, 89], B=2, T=300, d=256),
    "pagegram_B1_T700_d100": small_wl(1, pages=[53, 59], B=1, T=700, d=100),
    "pagegram_nosigns_B5_T1": small_wl(1, use_signs=0, pages=[7, 7], B=5, T=1, d=128),
    "engram_B4_T2_d64": small_wl(2, B=4, T=2, d=64),
    "orders_1to4_K2_B2_T513_d520": small_wl(1, K=2, S=4, n_min=1, n_max=4,
                                            pages=[5, 7, 11, 13], B=2, T=513, d=520),
    # one and two K stages (E = 64, 128)
    "one_slot_K1_B2_T300_d192": small_wl(1, K=1, n_min=2, n_max=2, pages=[97], B=2, T=300,
                                         d=192),
    "two_slots_K2_B1_T257_d256": small_wl(1, K=2, n_min=3, n_max=3, pages=[53], B=1, T=257,
                                          d=256),
}


def decode_signs(z0, z1):
    """Sign words from the two lane-half words of a record: element
    16 st + 8 h + 2 q (+1) sits at bit 15 - s (31 - s) of word h, s = 4 st + q."""
    z = (np.asarray(z0, np.uint64), np.asarray(z1, np.uint64))
    sw = np.zeros(np.shape(z0), dtype=np.uint64)
    for h in range(2):
        for st in range(4):
            for q in range(4):
                s = 4 * st + q
                e = 16 * st + 8 * h + 2 * q
                sw |= ((z[h] >> np.uint64(15 - s)) & np.uint64(1)) << np.uint64(e)
                sw |= ((z[h] >> np.uint64(31 - s)) & np.uint64(1)) << np.uint64(e + 1)
    return sw


def records(c, status=None):
    rec = torch.empty(pg.records_bytes(c.layout, c.N), dtype=torch.uint8, device=c.dev)
    pg.pg_index_records(c.layout, c.tokens, c.cmap, rec, dev_status=status)
    return rec


@pytest.mark.parametrize("name", list(CASES))
def test_records_decode_to_index_rows_and_signs(name):
    print(f"[gathered] records {name}", flush=True)
    c = Case(CASES[name])
    rec = records(c)
    idx = c.run_index()
    torch.cuda.synchronize()
    OK = c.O * c.K
    words = rec.view(torch.int32).cpu().numpy().view(np.uint32).reshape(OK, c.N, 4)
    rows = idx["rows"].cpu().numpy().reshape(c.N, OK)
    signs = idx["signs"].cpu().numpy().view(np.uint64).reshape(c.N, OK)
    assert np.array_equal(words[:, :, 0].T.astype(np.int64), rows)
    assert np.array_equal(decode_signs(words[:, :, 1], words[:, :, 2]).T, signs)
    assert (words[:, :, 3] == 0).all()
    if c.N <= 4096:
        ref = oracle.index(c.lay_d, c.tokens_np, c.cmap_np, c.pad)
        assert np.array_equal(rows, ref["rows"].reshape(c.N, OK))
        assert np.array_equal(signs, ref["signs"].reshape(c.N, OK))


@pytest.mark.parametrize("name", list(CASES))
def test_gathered_projection_equals_two_stage(name):
    print(f"[gathered] projection {name}", flush=True)
    c = Case(CASES[name])
    rec = records(c)
    e = c.run_index_gather()
    for inc in (0, 1):
        f = c.fuse(increment_only=inc)
        want = c.run_project(e, increment_only=inc)
        got = c.out_buffer()
        pg.pg_project_gathered(c.layout, c.table, f, rec, c.B, c.T, c.W, c.resid, got)
        fwd = c.run_forward(increment_only=inc)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), inc
        assert torch.equal(fwd.view(torch.uint8), want.view(torch.uint8)), inc
    # no residual: the increment alone
    got = c.out_buffer()
    pg.pg_project_gathered(c.layout, c.table, c.fuse(), rec, c.B, c.T, c.W, None, got)
    want = c.run_project(e, increment_only=1)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))


def test_records_flag_out_of_range_tokens():
    wl = small_wl(1, pages=[11, 13], B=2, T=16, d=64)
    toks = synth.tokens(configs.with_tokens(wl, 2, 16))
    toks[0, 3] = -5
    toks[1, 7] = wl["vocab"] + 3
    c = Case(wl, tokens=toks)
    st = torch.zeros(1, dtype=torch.int32, device=c.dev)
    rec = records(c, status=st)
    torch.cuda.synchronize()
    ref = oracle.index(c.lay_d, toks, c.cmap_np, c.pad)
    assert st.item() == 1
    words = rec.view(torch.int32).cpu().numpy().view(np.uint32).reshape(c.O * c.K, c.N, 4)
    assert np.array_equal(words[:, :, 0].T.astype(np.int64), ref["rows"].reshape(c.N, -1))


def test_forward_flags_out_of_range_tokens_on_the_gathered_path():
    wl = small_wl(1, pages=[11, 13], B=2, T=40, d=64)
    toks = synth.tokens(configs.with_tokens(wl, 2, 40))
    toks[0, 5] = -1
    toks[1, 39] = wl["vocab"]
    c = Case(wl, tokens=toks)
    f = c.fuse()
    ws = torch.empty(pg.pg_workspace_size(c.layout, f, c.B, c.T), dtype=torch.uint8,
                     device=c.dev)
    st = torch.zeros(1, dtype=torch.int32, device=c.dev)
    out = c.out_buffer()
    pg.pg_forward(c.layout, c.table, f, c.tokens, c.cmap, c.W, c.resid, out, ws, dev_status=st)
    e = c.run_index_gather()
    want = c.run_project(e)
    torch.cuda.synchronize()
    assert st.item() == 1
    assert torch.equal(out.view(torch.uint8), want.view(torch.uint8))
    ref = c.oracle_scalar(np.arange(c.N))["out"]
    assert rel_err(out.double().cpu().numpy(), ref) < 2e-2


def test_gathered_rejects_other_tables_and_gates():
    c = Case(small_wl(3, r=64, pages=[31, 37], B=2, T=20, d=128))      # NF4 table
    rec = torch.empty(pg.records_bytes(c.layout, c.N), dtype=torch.uint8, device=c.dev)
    pg.pg_index_records(c.layout, c.tokens, c.cmap, rec)
    out = c.out_buffer()
    with pytest.raises(pg.PagegramError):
        pg.pg_project_gathered(c.layout, c.table, c.fuse(), rec, c.B, c.T, c.W, c.resid, out)
    c = Case(small_wl(1, r=32, pages=[31, 37], B=2, T=20, d=128))      # 32-element rows
    with pytest.raises(pg.PagegramError):
        pg.pg_index_records(c.layout, c.tokens, c.cmap, rec)
