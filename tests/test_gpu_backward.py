"""GPU parity of the backward pass and the sparse row-wise table update
against the oracle (oracle/backward.py).

Bit-exact: the distinct touched rows (ascending) and their count. Within
tolerance (fp32 accumulation of bf16 products vs float64): de, dW and the
per-row gradients; the optimiser state after several steps and a flush.
"""
import numpy as np
import pytest
import torch

import hashed_head_gram_amd as pg
import oracle
from oracle import backward as ob
from synth import configs
from tests.gpu_inputs import Case, rel_err
from tests.test_gpu_parity import small_wl

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _bf16(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(torch.bfloat16)


def _run_backward(c, dy, g):
    idx = c.run_index()
    e = c.run_index_gather()
    N, E, d = c.N, c.E, c.d
    L = N * c.O * c.K
    f = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, d, g=g)
    ws = torch.empty(pg.pg_backward_workspace_size(c.layout, f, c.B, c.T), dtype=torch.uint8,
                     device=c.dev)
    dW = torch.empty(d, E, dtype=torch.float32, device=c.dev)
    de = torch.empty(N, E, dtype=torch.float32, device=c.dev)
    urows = torch.full((L,), -1, dtype=torch.int64, device=c.dev)
    ugrad = torch.empty(L, c.r, dtype=torch.float32, device=c.dev)
    nu = torch.zeros(1, dtype=torch.int64, device=c.dev)
    pg.pg_backward_scalar(c.layout, f, idx["rows"], idx["signs"], e, dy, c.W, c.B, c.T, dW, de,
                          urows, ugrad, nu, ws)
    torch.cuda.synchronize()
    n = int(nu.item())
    return dict(idx=idx, e=e, dW=dW, de=de, urows=urows[:n], ugrad=ugrad[:n], n=n, L=L)


BACKWARD_CASES = {
    "pagegram_K4_S4_r16_T100": small_wl(1, K=4, S=4, r=16, pages=[7, 5], B=2, T=100, d=128),
    "engram_K4_r32_T77": small_wl(2, K=4, r=32, head_rows=[11, 13, 17, 19, 23, 29, 31, 37],
                                  B=3, T=77, d=192),
    "pagegram_nosigns_K8_r64": small_wl(1, use_signs=0, pages=[31, 29], B=2, T=64, d=64),
}


@pytest.mark.parametrize("name", list(BACKWARD_CASES))
def test_backward_matches_oracle(name):
    wl = BACKWARD_CASES[name]
    print(f"[backward] {name}", flush=True)
    c = Case(wl)
    rng = np.random.default_rng(17)
    dy_np = rng.standard_normal((c.N, c.d)).astype(np.float32)
    dy = _bf16(dy_np, c.dev)
    g = 0.5
    out = _run_backward(c, dy, g)
    e64 = out["e"].double().cpu().numpy()
    W64 = c.W.double().cpu().numpy()
    dy64 = dy.double().cpu().numpy()
    dW_ref, de_ref = ob.backward_dense(e64, W64, g, dy64)
    err_de = rel_err(out["de"].cpu().numpy(), de_ref)
    err_dW = rel_err(out["dW"].cpu().numpy(), dW_ref)
    print(f"[backward] {name} rel err de {err_de:.2e} dW {err_dW:.2e}")
    assert err_de < TOL and err_dW < TOL
    rows = out["idx"]["rows"].cpu().numpy()
    signs = out["idx"]["signs"].cpu().numpy().view(np.uint64)
    ur_ref, gr_ref = ob.row_gradients(c.lay_d, rows, signs, de_ref)
    assert out["n"] == len(ur_ref)
    assert np.array_equal(out["urows"].cpu().numpy(), ur_ref)
    err = rel_err(out["ugrad"].cpu().numpy(), gr_ref)
    print(f"[backward] {name} n_unique {out['n']} of {out['L']} lookups, row-grad rel err {err:.2e}")
    assert err < TOL


def test_backward_full_size_sampled():
    """The 200M PageGram workload (16,384 tokens, 262,144 lookups): the set of
    touched rows exactly, and sampled rows of de, dW and the row gradients."""
    wl = configs.workload(1)
    c = Case(wl)
    rng = np.random.default_rng(23)
    dy_np = (rng.standard_normal((c.N, c.d)) * 0.1).astype(np.float32)
    dy = _bf16(dy_np, c.dev)
    out = _run_backward(c, dy, 0.5)
    rows = out["idx"]["rows"].cpu().numpy()
    ur = np.unique(rows)
    assert out["n"] == len(ur)
    assert np.array_equal(out["urows"].cpu().numpy(), ur)
    e64 = out["e"].double().cpu().numpy()
    W64 = c.W.double().cpu().numpy()
    dy64 = dy.double().cpu().numpy()
    tok = rng.choice(c.N, size=64, replace=False)
    de_ref = 0.5 * (dy64[tok] @ W64)
    err_de = rel_err(out["de"].cpu().numpy()[tok], de_ref)
    cols = rng.choice(c.E, size=32, replace=False)
    dW_ref = 0.5 * (dy64.T @ e64[:, cols])
    err_dW = rel_err(out["dW"].cpu().numpy()[:, cols], dW_ref)
    print(f"[backward] full size rel err de {err_de:.2e} dW {err_dW:.2e}")
    assert err_de < TOL and err_dW < TOL
    # row gradients of sampled rows from the device de (exact lookup lists)
    de_dev = out["de"].double().cpu().numpy()
    signs = out["idx"]["signs"].cpu().numpy().view(np.uint64)
    pick = rng.choice(len(ur), size=200, replace=False)
    sel = np.isin(rows, ur[pick])
    N, O, K = rows.shape
    r = c.r
    sv = oracle.sign_vectors(signs, r).reshape(N, O, K, r)
    contrib = de_dev.reshape(N, O, K, r) * sv
    want = np.zeros((len(pick), r))
    pos = {int(u): i for i, u in enumerate(ur[pick])}
    for (t, n, k) in zip(*np.nonzero(sel)):
        want[pos[int(rows[t, n, k])]] += contrib[t, n, k]
    got = out["ugrad"].cpu().numpy()[pick]
    assert rel_err(got, want) < 1e-5


def test_row_rms_steps_and_flush_match_oracle():
    wl = BACKWARD_CASES["pagegram_K4_S4_r16_T100"]
    c = Case(wl)
    R, r = c.R, c.r
    lr, beta2, wd, eps = 0.05, 0.95, 0.2, 1e-8
    table = torch.zeros(R, r, dtype=torch.float32, device=c.dev)
    vhat = torch.zeros(R, dtype=torch.float32, device=c.dev)
    last = torch.zeros(R, dtype=torch.int64, device=c.dev)
    th_ref, v_ref, last_ref = np.zeros((R, r)), np.zeros(R), np.zeros(R, np.int64)
    rng = np.random.default_rng(29)
    for step in range(1, 5):
        # a different token window each step, so rows are skipped and replayed
        toks = c.tokens_np.copy()
        toks = np.roll(toks, 13 * step, axis=1)
        cs = Case(wl, tokens=toks)
        dy = _bf16(rng.standard_normal((cs.N, cs.d)), cs.dev)
        out = _run_backward(cs, dy, 1.0)
        pg.pg_row_rms_step(c.layout, out["urows"], out["ugrad"],
                           torch.tensor([out["n"]], dtype=torch.int64, device=c.dev),
                           out["n"], table, vhat, last, step, lr, beta2, wd, eps)
        th_ref, v_ref, last_ref = ob.rms_step_sparse(
            th_ref, v_ref, last_ref, out["urows"].cpu().numpy(),
            out["ugrad"].double().cpu().numpy(), step, lr, beta2, wd, eps)
        torch.cuda.synchronize()
        assert np.array_equal(last.cpu().numpy(), last_ref)
        assert rel_err(table.cpu().numpy(), th_ref) < 1e-5
        assert rel_err(vhat.cpu().numpy(), v_ref) < 1e-5
    pg.pg_row_rms_flush(c.layout, table, vhat, last, 6, lr, beta2, wd)
    th_ref, v_ref, last_ref = ob.rms_flush(th_ref, v_ref, last_ref, 6, lr, beta2, wd)
    torch.cuda.synchronize()
    assert (last.cpu().numpy() == 6).all()
    assert rel_err(table.cpu().numpy(), th_ref) < 1e-5
    assert rel_err(vhat.cpu().numpy(), v_ref) < 1e-5


def test_backward_rejects_unsupported_shapes():
    wl = small_wl(1, pages=[7, 5], B=2, T=8, d=100)       # d not a multiple of 64
    c = Case(wl)
    f = pg.make_fuse(pg.PG_GATE_SCALAR, pg.PG_BF16, c.d, g=0.5)
    with pytest.raises(pg.PagegramError):
        pg.pg_backward_workspace_size(c.layout, f, c.B, c.T)
