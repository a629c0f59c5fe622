"""pg_forward_noalloc, the entry point for callers that cannot allocate device
memory: pg_forward with its workspace in the library's static device array.

GPU: it runs the same kernels as pg_forward, so its output must equal
pg_forward's (caller workspace) bit for bit. Each case makes two calls in a
row, the second on a smaller input, so the second reads a scratch array
that still holds the first call's contents; both forward paths are covered
(the gathered projection of 64-element bf16 rows under the scalar gate, and
the two-kernel path with the NF4 table and with the Engram gate). CPU: the
size limit and argument checks return their errors before any launch.
"""
import ctypes

import pytest
import torch

import hashed_head_gram_amd as pg
from synth import configs
from tests.gpu_inputs import Case, layout_of
from tests.test_gpu_parity import small_wl

FAKE = 1 << 40          # aligned, never dereferenced by the host-side checks

PAIRS = {
    # gathered projection: the 200M PageGram workload, then a ragged batch
    "pagegram200m_then_B3_T700": (configs.workload(1),
                                  configs.with_tokens(configs.workload(1), 3, 700)),
    # two-kernel path, NF4 table: e and the projection in the scratch array
    "nf4_B2_T100_then_B1_T33": (small_wl(3, r=64, pages=[31, 37], B=2, T=100, d=128),
                                small_wl(3, r=64, pages=[31, 37], B=1, T=33, d=128)),
    # two-kernel path, Engram gate: e, v, the partial sums and the gates
    "engram_gate_B2_T45_then_B1_T20": (
        small_wl(4, K=4, r=24, head_rows=[101, 103, 107, 109, 113, 127, 131, 137], B=2,
                 T=45, d=256, M=2, gamma="random"),
        small_wl(4, K=4, r=24, head_rows=[101, 103, 107, 109, 113, 127, 131, 137], B=1,
                 T=20, d=256, M=2, gamma="random")),
}


def _with_workspace(c):
    f = c.fuse()
    ws = torch.empty(max(pg.pg_workspace_size(c.layout, f, c.B, c.T), 256),
                     dtype=torch.uint8, device=c.dev)
    out = c.out_buffer()
    pg.pg_forward(c.layout, c.table, f, c.tokens, c.cmap, c.W, c.resid, out, ws)
    return out


def _no_alloc(c, status=None):
    out = c.out_buffer()
    out.fill_(7.0)
    pg.pg_forward_noalloc(c.layout, c.table, c.fuse(), c.tokens, c.cmap, c.W, c.resid, out,
                          dev_status=status)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_equals_forward_twice(name):
    big_wl, small = PAIRS[name]
    big = Case(big_wl)
    print(f"[no_alloc] {name}: first call, {big.N} tokens", flush=True)
    st = torch.zeros(1, dtype=torch.int32, device=big.dev)
    got1 = _no_alloc(big, st)
    want1 = _with_workspace(big)
    torch.cuda.synchronize()
    assert torch.equal(got1.view(torch.uint8), want1.view(torch.uint8))
    assert st.item() == 0
    sm = Case(small)
    assert sm.N < big.N
    print(f"[no_alloc] {name}: second call, {sm.N} tokens", flush=True)
    got2 = _no_alloc(sm)
    want2 = _with_workspace(sm)
    torch.cuda.synchronize()
    assert torch.equal(got2.view(torch.uint8), want2.view(torch.uint8))


@pytest.mark.gpu
def test_noalloc_back_to_back_on_one_stream():
    # both calls enqueued before either is waited for: stream order alone
    # keeps the second call's use of the scratch array after the first's
    big = Case(PAIRS["pagegram200m_then_B3_T700"][0])
    sm = Case(PAIRS["pagegram200m_then_B3_T700"][1])
    print("[no_alloc] back to back", flush=True)
    got_big = _no_alloc(big)
    got_sm = _no_alloc(sm)
    want_big = _with_workspace(big)
    want_sm = _with_workspace(sm)
    torch.cuda.synchronize()
    assert torch.equal(got_big.view(torch.uint8), want_big.view(torch.uint8))
    assert torch.equal(got_sm.view(torch.uint8), want_sm.view(torch.uint8))


def test_noalloc_host_side_limits():
    L = pg.lib()
    by = ctypes.byref
    wl = configs.workload(1)
    lay = layout_of(wl)
    R = pg.pg_layout_rows(lay)
    tab = pg.make_table(pg.PG_BF16, FAKE, R)
    f = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, 768)
    assert pg.NOALLOC_SCRATCH_BYTES == 64 << 20
    # 8 x 2048 tokens need 32 MiB; 8 x 8192 need 128 MiB: beyond the array
    assert pg.pg_workspace_size(lay, f, 8, 2048) <= pg.NOALLOC_SCRATCH_BYTES
    assert pg.pg_workspace_size(lay, f, 8, 8192) > pg.NOALLOC_SCRATCH_BYTES
    assert L.pg_forward_noalloc(by(lay), by(tab), by(f), FAKE, 8, 8192, FAKE, 50304, FAKE,
                                FAKE, FAKE, None, None) == pg.PG_ERANGE
    # the Engram gate's workspace of the 27B fusion workload does not fit either
    g = pg.make_fuse(pg.PG_GATE_ENGRAM, pg.PG_BF16, 2560, M=4, gamma_h=FAKE, gamma_k=FAKE,
                     gamma_u=FAKE, conv_w=FAKE)
    wl5 = configs.workload(4)
    lay5 = layout_of(wl5)
    tab5 = pg.make_table(pg.PG_BF16, FAKE, pg.pg_layout_rows(lay5))
    assert L.pg_forward_noalloc(by(lay5), by(tab5), by(g), FAKE, 32, 4096, FAKE, 128000,
                                FAKE, FAKE, FAKE, None, None) == pg.PG_ERANGE
    # pg_forward's other checks apply unchanged
    assert L.pg_forward_noalloc(by(lay), by(tab), by(f), FAKE, 8, 2048, FAKE, 50304, None,
                                FAKE, FAKE, None, None) == pg.PG_EINVAL
    assert L.pg_forward_noalloc(by(lay), by(tab), by(f), None, 0, 2048, None, 0, None,
                                None, None, None, None) == pg.PG_OK
