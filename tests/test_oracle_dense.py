"""Pins of the oracle's gather, NF4, projection and fusion stages.

  * the flat-table special case K=1, S=1, r=d (PageGram §2.1 eq. for e_t vs
    the §3.1 row formula): with W = [I_d I_d] the multi-head path collapses to
    e_t = sum_n s_n * T[h_n];
  * one-hot projections read back single elements, which fixes the concat
    order (order outer, head inner; Engram notes §3.2);
  * a zero table leaves the residual unchanged (PageGram §9.4, check 3);
  * NF4 byte arithmetic (PageGram §2.3, §3.3: 34 B per row, 120 rows and
    4080 B per 4 KiB page at S=15, 1088 B and 3 pages per 4 KiB block at S=4);
    zero-row fidelity and the quantisation error bound (§9.4, check 5);
  * projection against explicit loops; causal conv against torch conv1d;
    context-gate closed forms (alpha = sigmoid(sqrt(d)) when h is parallel
    to k; alpha = 1/2 when W_K = 0); causality with the conv included.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import pagegram as og


def lay(kind="pagegram", K=4, S=4, r=16, P=11, primes=None, use_signs=1,
        seed=77):
    return dict(kind=kind, n_min=2, n_max=3, K=K, S=S, r=r, pages=[P, P],
                head_rows=list(primes or [P * S] * (2 * K)), hash_seed=seed,
                use_signs=use_signs)


def rand_table(R, r, seed=0):
    return np.random.default_rng(seed).normal(0, 0.02, (R, r)).astype(np.float32)


def test_flat_special_case():
    d = 24
    L = lay(K=1, S=1, r=d, P=53)
    _, R = og.layout_bases(L)
    T = rand_table(R, d)
    W = np.concatenate([np.eye(d), np.eye(d)], axis=1)      # [d, 2d]
    toks = np.random.default_rng(1).integers(0, 400, size=(2, 50))
    x = np.random.default_rng(2).normal(size=(100, d))
    res = oracle.forward_scalar(L, 400, toks, np.arange(400), "f32",
                                lambda r: T[r], W, 0.5, None)
    full = oracle.forward_scalar(L, 400, toks, np.arange(400), "f32",
                                 lambda r: T[r], W, 0.5, lambda p: x[p])
    rows, signs = res["index"]["rows"], res["index"]["signs"]
    flat = np.zeros((100, d))
    for n in range(2):
        s = 1.0 - 2.0 * ((signs[:, n, 0, 0][:, None] >> np.arange(d).astype(
            np.uint64)) & np.uint64(1)).astype(np.float64)
        flat += s * T[rows[:, n, 0]].astype(np.float64)
    # increment: exactly g * (s_2 T[h_2] + s_3 T[h_3]) (one rounding each)
    np.testing.assert_array_equal(res["out"], 0.5 * flat)
    np.testing.assert_allclose(full["out"], x + 0.5 * flat, rtol=0, atol=1e-15)
    # K=1, S=1 rows are base_n + p_n: the flat hash into P_n rows
    assert np.array_equal(rows[:, 0, 0], res["index"]["pages"][:, 0])
    assert np.array_equal(rows[:, 1, 0], 53 + res["index"]["pages"][:, 1])


def test_concat_order_by_one_hot_projection():
    L = lay(K=3, S=2, r=8, P=5)
    _, R = og.layout_bases(L)
    T = rand_table(R, 8, seed=3)
    E = 2 * 3 * 8
    toks = np.random.default_rng(4).integers(0, 90, size=(1, 20))
    idx = oracle.index(L, toks, np.arange(90), 90)
    for (n, k, j) in [(0, 0, 0), (0, 2, 7), (1, 0, 3), (1, 2, 5)]:
        W = np.zeros((1, E))
        W[0, (n * 3 + k) * 8 + j] = 1.0
        res = oracle.forward_scalar(L, 90, toks, np.arange(90), "f32",
                                    lambda r: T[r], W, 1.0, None)
        sbit = (idx["signs"][:, n, k, 0] >> np.uint64(j)) & np.uint64(1)
        want = (1.0 - 2.0 * sbit) * T[idx["rows"][:, n, k], j]
        np.testing.assert_array_equal(res["out"][:, 0], want)


def test_projection_against_loops():
    rng = np.random.default_rng(5)
    e = rng.normal(size=(3, 7))
    W = rng.normal(size=(4, 7))
    y = og.project(e, W)
    for t in range(3):
        for o in range(4):
            acc = 0.0
            for i in range(7):
                acc += W[o, i] * e[t, i]
            assert abs(y[t, o] - acc) < 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16", "nf4"])
def test_zero_table_leaves_residual(dtype):
    L = lay(K=8, S=4, r=64, P=17)
    _, R = og.layout_bases(L)
    if dtype == "nf4":
        fetch = lambda r: (np.zeros((len(r), 32), np.uint8),  # noqa: E731
                           np.zeros(len(r), np.float16))
    elif dtype == "bf16":
        fetch = lambda r: np.zeros((len(r), 64), np.uint16)   # noqa: E731
    else:
        fetch = lambda r: np.zeros((len(r), 64), np.float32)  # noqa: E731
    toks = np.random.default_rng(6).integers(0, 300, size=(2, 40))
    x = np.random.default_rng(7).normal(size=(80, 16))
    W = np.random.default_rng(8).normal(size=(16, 1024))
    res = oracle.forward_scalar(L, 300, toks, np.arange(300), dtype, fetch, W,
                                0.5, lambda p: x[p])
    assert np.array_equal(res["out"], x)


def test_nf4_format_arithmetic():
    row_bytes = 64 * 4 // 8 + 16 // 8
    assert row_bytes == 34
    assert 4096 // row_bytes == 120
    assert 8 * 15 * row_bytes == 4080 <= 4096
    page_s4 = 8 * 4 * row_bytes
    assert page_s4 == 1088
    assert 3 * page_s4 <= 4096 < 4 * page_s4
    assert abs(4096 / (3 * page_s4) - 1.255) < 1e-3     # about 25% overhead


def test_nf4_codebook_shape():
    cb = og.nf4_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[-1] == 1.0 and cb[7] == 0.0
    assert (cb < 0).sum() == 7 and (cb > 0).sum() == 8
    # levels are standard-normal quantiles: mapped back through the normal
    # CDF (rescaled by the outer quantile), positive and negative levels sit
    # at evenly spaced probabilities.
    from scipy.stats import norm
    z = norm.ppf(0.5 * ((1 - 1 / 30) + (1 - 1 / 32)))
    pp = norm.cdf(cb[8:].astype(np.float64) * z)
    pn = norm.cdf(-cb[:7].astype(np.float64) * z)
    assert np.allclose(np.diff(pp), pp[1] - pp[0], atol=1e-6)
    assert np.allclose(np.diff(pn), pn[1] - pn[0], atol=1e-6)


def test_nf4_nibble_order_and_zero_row():
    codes = np.array([[0x21, 0xF0] + [0x77] * 30], dtype=np.uint8)
    q = og.nf4_unpack(codes, 64)
    assert q[0, :4].tolist() == [1, 2, 0, 15]
    packed, scale = og.nf4_quantize(np.zeros((2, 64)))
    assert (scale == 0).all()
    assert np.array_equal(og.nf4_dequantize(packed, scale, 64), np.zeros((2, 64)))


def test_nf4_quantisation_error_bound_and_round_trip():
    rng = np.random.default_rng(10)
    x = rng.normal(0, 0.02, size=(500, 64))
    packed, scale = og.nf4_quantize(x)
    y = og.nf4_dequantize(packed, scale, 64)
    cb = og.nf4_codebook().astype(np.float64)
    gap = np.max(np.diff(cb)) / 2
    s = scale.astype(np.float64)
    absmax = np.abs(x).max(axis=1)
    bound = s * gap + np.abs(absmax - s) + 1e-12
    assert np.all(np.abs(x - y).max(axis=1) <= bound)
    # rows made of codebook levels times a representable scale round-trip
    q = rng.integers(0, 16, size=(50, 64))
    q[:, 0] = 15                                         # absmax = scale
    sc = np.float16(0.0625)
    vals = cb[q] * float(sc)
    packed, scale = og.nf4_quantize(vals)
    assert (scale == sc).all()
    assert np.array_equal(og.nf4_unpack(packed, 64), q)


def test_gather_stored_matches_exact_gather():
    L = lay(K=8, S=4, r=64, P=9)
    _, R = og.layout_bases(L)
    rng = np.random.default_rng(11)
    toks = rng.integers(0, 500, size=(2, 60))
    idx = oracle.index(L, toks, np.arange(500), 500)
    f32 = rand_table(R, 64, seed=12)
    bf = (f32.view(np.uint32) >> 16).astype(np.uint16)
    codes = rng.integers(0, 256, size=(R, 32)).astype(np.uint8)
    scales = rng.uniform(0.01, 0.1, size=R).astype(np.float16)
    for dt, fetch in (("f32", lambda r: f32[r]), ("bf16", lambda r: bf[r]),
                      ("nf4", lambda r: (codes[r], scales[r]))):
        ex = og.gather(L, dt, fetch, idx["rows"], idx["signs"])
        st = og.gather_stored(L, dt, fetch, idx["rows"], idx["signs"])
        if dt == "f32":
            np.testing.assert_array_equal(st.astype(np.float64), ex)
        else:
            stf = (st.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            if dt == "bf16":
                np.testing.assert_array_equal(stf, ex)
            else:
                # one fp32 and one bf16 rounding: within 2^-8 relative
                assert np.all(np.abs(stf - ex) <= np.abs(ex) * 2.0 ** -8)
                assert np.array_equal(np.signbit(stf[ex != 0]),
                                      np.signbit(ex[ex != 0]))


# ---------------------------------------------------------------------------
# Engram fusion


def engram_case(d=16, M=2, Bs=2, Ts=24, seed=0, K=2, r=8, zero_table=False,
                zero_wk=False, conv=None, gammas=True):
    L = lay(kind="engram", K=K, r=r, primes=[13] * (2 * K))
    _, R = og.layout_bases(L)
    rng = np.random.default_rng(seed)
    Tb = (np.zeros((R, r), np.float32) if zero_table
          else rng.normal(0, 0.5, (R, r)).astype(np.float32))
    E = 2 * K * r
    W = rng.normal(0, 0.3, ((1 + M) * d, E))
    if zero_wk:
        W[d:] = 0
    h = rng.normal(size=(M, Bs * Ts, d))
    g = [1.0 + rng.normal(0, 0.2, d) if gammas else np.ones(d) for _ in range(3)]
    cw = conv if conv is not None else rng.normal(0, 0.5, (d, 4))
    toks = rng.integers(0, 60, size=(Bs, Ts))
    return dict(L=L, T=Tb, W=W, h=h, g=g, cw=cw, toks=toks, d=d, M=M, Bs=Bs,
                Ts=Ts)


def run_oracle(c, positions=None, with_resid=True):
    return oracle.forward_engram(
        c["L"], 60, c["toks"], np.arange(60), "f32", lambda r: c["T"][r],
        c["W"], c["d"], c["M"], c["g"][0], c["g"][1], c["g"][2], c["cw"], 3,
        1e-6, lambda m, f: c["h"][m, f], positions=positions,
        with_resid=with_resid)


def torch_reference(c):
    """Whole-batch fp64 computation with torch's conv1d as the conv."""
    idx = oracle.index(c["L"], c["toks"], np.arange(60), 60)
    e = og.gather(c["L"], "f32", lambda r: c["T"][r], idx["rows"], idx["signs"])
    d, M, Bs, Ts = c["d"], c["M"], c["Bs"], c["Ts"]
    W = torch.tensor(c["W"])
    e = torch.tensor(e)
    v = e @ W[:d].T
    gh, gk, gu = (torch.tensor(x) for x in c["g"])

    def rms(x, g):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + 1e-6) * g
    outs = []
    for m in range(M):
        k = e @ W[d * (1 + m):d * (2 + m)].T
        h = torch.tensor(c["h"][m])
        alpha = torch.sigmoid((rms(h, gh) * rms(k, gk)).sum(-1) / math.sqrt(d))
        u = alpha[:, None] * v
        z = rms(u, gu).reshape(Bs, Ts, d).transpose(1, 2)       # [B, d, T]
        w = torch.tensor(c["cw"]).reshape(d, 1, 4)
        y = torch.nn.functional.conv1d(
            torch.nn.functional.pad(z, (9, 0)), w, groups=d, dilation=3)
        Y = torch.nn.functional.silu(y).transpose(1, 2).reshape(Bs * Ts, d) + u
        outs.append(Y.numpy())
    return np.stack(outs)


def test_engram_fusion_matches_torch_conv1d():
    c = engram_case()
    got = run_oracle(c, with_resid=False)["out"]
    np.testing.assert_allclose(got, torch_reference(c), rtol=1e-12, atol=1e-12)


def test_engram_fusion_residual():
    c = engram_case(seed=3)
    pos = [0, 5, 30, 47]
    a = run_oracle(c, positions=pos)["out"]
    b = run_oracle(c, positions=pos, with_resid=False)["out"]
    np.testing.assert_allclose(a - b, c["h"][:, pos], rtol=0, atol=1e-12)


def test_engram_zero_table_is_identity():
    # zero table: k = 0 gives alpha = 1/2, u~ = 0, Y = SiLU(conv(0)) + 0 = 0.
    c = engram_case(zero_table=True)
    out = run_oracle(c)["out"]
    assert np.array_equal(out, c["h"])


def test_engram_gate_closed_forms():
    d = 16
    rng = np.random.default_rng(1)
    k = rng.normal(size=d)
    # h parallel to k, unit gains: RMSNorm(h).RMSNorm(k) = d (up to eps)
    hn = og.rmsnorm(3.0 * k, np.ones(d), 0.0)
    kn = og.rmsnorm(k, np.ones(d), 0.0)
    assert abs(og.sigmoid(np.dot(hn, kn) / math.sqrt(d)) - og.sigmoid(4.0)) < 1e-12
    # RMSNorm output has unit mean square and is scale invariant
    assert abs(np.mean(kn ** 2) - 1.0) < 1e-12
    assert np.allclose(og.rmsnorm(7.5 * k, np.ones(d), 0.0), kn)
    # W_K = 0: alpha = 1/2 exactly; last conv tap only: conv is the identity
    cw = np.zeros((16, 4))
    cw[:, 3] = 1.0
    c = engram_case(zero_wk=True, conv=cw, gammas=False)
    out = run_oracle(c, with_resid=False)["out"]
    idx = oracle.index(c["L"], c["toks"], np.arange(60), 60)
    e = og.gather(c["L"], "f32", lambda r: c["T"][r], idx["rows"], idx["signs"])
    u = 0.5 * (e @ c["W"][:16].T)
    z = og.rmsnorm(u, np.ones(16), 1e-6)
    want = og.silu(z) + u
    np.testing.assert_allclose(out[0], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out[1], want, rtol=1e-12, atol=1e-14)
    # first tap only: y_t = z_{t-9}, zero for t < 9 in each sequence
    cw = np.zeros((16, 4))
    cw[:, 0] = 1.0
    c2 = dict(c, cw=cw)
    out2 = run_oracle(c2, with_resid=False)["out"]
    zz = z.reshape(2, 24, 16)
    shifted = np.zeros_like(zz)
    shifted[:, 9:] = zz[:, :-9]
    want2 = og.silu(shifted.reshape(48, 16)) + u
    np.testing.assert_allclose(out2[0], want2, rtol=1e-12, atol=1e-14)


def test_engram_causality_with_conv():
    c = engram_case(seed=4)
    base = run_oracle(c)["out"]
    t_edit = 15
    c2 = dict(c)
    c2["toks"] = c["toks"].copy()
    c2["toks"][:, t_edit:] = (c["toks"][:, t_edit:] + 7) % 60
    h2 = c["h"].copy()
    h2[:, :, :] = c["h"]
    c2["h"] = h2
    other = run_oracle(c2)["out"]
    keep = (np.arange(c["Bs"] * c["Ts"]) % c["Ts"]) < t_edit
    assert np.array_equal(base[:, keep], other[:, keep])
    assert not np.allclose(base[:, ~keep], other[:, ~keep])


def test_scalar_path_causality():
    L = lay(K=4, S=4, r=16, P=64)
    _, R = og.layout_bases(L)
    T = rand_table(R, 16, seed=20)
    W = np.random.default_rng(21).normal(0, 0.05, (64, 128))
    rng = np.random.default_rng(22)
    toks = rng.integers(0, 1024, size=(1, 256))
    x = rng.normal(size=(256, 64))
    a = oracle.forward_scalar(L, 1024, toks, np.arange(1024), "f32",
                              lambda r: T[r], W, 0.5, lambda p: x[p])["out"]
    toks2 = toks.copy()
    toks2[0, 100:] = rng.integers(0, 1024, size=156)
    b = oracle.forward_scalar(L, 1024, toks2, np.arange(1024), "f32",
                              lambda r: T[r], W, 0.5, lambda p: x[p])["out"]
    assert np.array_equal(a[:100], b[:100])
    assert not np.allclose(a[100:], b[100:])
