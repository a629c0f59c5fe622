"""Pins of the backward / sparse-update oracle (oracle/backward.py).

Independent of the oracle's own formulas:
  * finite differences of the oracle's *forward* (the loss sum(dy * out) is
    linear in W and in the table, and with integer-valued inputs every
    difference is exact in float64), so dW, de and the table gradient are
    checked against the definition of a derivative;
  * PageGram §9.4 check 4: the sparse per-row gradient equals the dense
    table gradient (np.add.at over every lookup);
  * the lazy per-row optimiser with replayed decay equals the dense optimiser
    that visits every row every step with zero gradients (check 4), and one
    step from the zero state has its closed form.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ob


def _tiny_layout(kind="pagegram", K=3, S=2, r=8, P=5, use_signs=1):
    return dict(kind=kind, n_min=2, n_max=3, K=K, S=S, r=r, pages=[P, P],
                head_rows=[P * S + 1 + k for k in range(2 * K)], hash_seed=0x1234,
                use_signs=use_signs)


def _problem(lay, seed=0, B=2, T=6, V=11, d=4):
    rng = np.random.default_rng(seed)
    R = oracle.layout_bases(lay)[1]
    table = rng.integers(-4, 5, size=(R, lay["r"])).astype(np.float32)
    W = rng.integers(-3, 4, size=(d, 2 * lay["K"] * lay["r"])).astype(np.float64)
    tokens = rng.integers(0, V, size=(B, T))
    cmap = np.arange(V, dtype=np.int64)
    dy = rng.integers(-2, 3, size=(B * T, d)).astype(np.float64)
    return table, W, tokens, cmap, dy, V


def _loss(lay, table, W, tokens, cmap, V, dy, g):
    out = oracle.forward_scalar(lay, V, tokens, cmap, "f32", lambda rows: table[rows], W, g,
                                None)["out"]
    return float(np.sum(dy * out))


@pytest.mark.parametrize("kind", ["pagegram", "engram"])
def test_gradients_match_finite_differences(kind):
    lay = _tiny_layout(kind=kind)
    table, W, tokens, cmap, dy, V = _problem(lay)
    g = 0.5
    fw = oracle.forward_scalar(lay, V, tokens, cmap, "f32", lambda rows: table[rows], W, g, None)
    e = fw["e"]
    dW, de = ob.backward_dense(e, W, g, dy)
    base = _loss(lay, table, W, tokens, cmap, V, dy, g)
    # dW: every entry by a unit perturbation (the loss is linear in W)
    for (i, j) in [(0, 0), (1, 5), (3, 2 * lay["K"] * lay["r"] - 1), (2, 7)]:
        W2 = W.copy()
        W2[i, j] += 1.0
        assert _loss(lay, table, W2, tokens, cmap, V, dy, g) - base == dW[i, j]
    # table gradient: sparse rows against unit perturbations of the table
    idx = fw["index"]
    urows, grads = ob.row_gradients(lay, idx["rows"], idx["signs"], de)
    for u in list(urows[:3]) + [urows[-1]]:
        for j in (0, lay["r"] - 1):
            t2 = table.copy()
            t2[u, j] += 1.0
            diff = _loss(lay, t2, W, tokens, cmap, V, dy, g) - base
            assert diff == grads[list(urows).index(u), j]
    # an untouched row has zero gradient
    R = oracle.layout_bases(lay)[1]
    untouched = sorted(set(range(R)) - set(urows.tolist()))
    assert untouched
    t2 = table.copy()
    t2[untouched[0], 0] += 1.0
    assert _loss(lay, t2, W, tokens, cmap, V, dy, g) == base


@pytest.mark.parametrize("use_signs", [0, 1])
def test_sparse_gradient_equals_dense(use_signs):
    lay = _tiny_layout(use_signs=use_signs)
    table, W, tokens, cmap, dy, V = _problem(lay, seed=3)
    fw = oracle.forward_scalar(lay, V, tokens, cmap, "f32", lambda rows: table[rows], W, 1.0, None)
    _, de = ob.backward_dense(fw["e"], W, 1.0, dy)
    idx = fw["index"]
    urows, grads = ob.row_gradients(lay, idx["rows"], idx["signs"], de)
    R = oracle.layout_bases(lay)[1]
    G = ob.dense_table_gradient(lay, R, idx["rows"], idx["signs"], de)
    assert np.array_equal(G[urows], grads)
    mask = np.ones(R, bool)
    mask[urows] = False
    assert not G[mask].any()
    assert np.all(np.diff(urows) > 0)


def test_lazy_update_equals_dense_update():
    rng = np.random.default_rng(5)
    R, r = 12, 6
    eta, beta2, lam, eps = 0.07, 0.95, 0.3, 1e-8
    theta_d = rng.normal(size=(R, r))
    v_d = np.zeros(R)
    theta_s, v_s, last = theta_d.copy(), v_d.copy(), np.zeros(R, np.int64)
    for step in range(1, 9):
        touched = np.sort(rng.choice(R, size=int(rng.integers(1, 5)), replace=False))
        grads = rng.normal(size=(len(touched), r))
        G = np.zeros((R, r))
        G[touched] = grads
        theta_d, v_d = ob.rms_step_dense(theta_d, v_d, G, eta, beta2, lam, eps)
        theta_s, v_s, last = ob.rms_step_sparse(theta_s, v_s, last, touched, grads, step,
                                               eta, beta2, lam, eps)
    theta_f, v_f, last_f = ob.rms_flush(theta_s, v_s, last, 8, eta, beta2, lam)
    assert np.allclose(theta_f, theta_d, rtol=1e-12, atol=1e-14)
    assert np.allclose(v_f, v_d, rtol=1e-12, atol=1e-300)
    assert (last_f == 8).all()


def test_one_step_closed_form():
    eta, beta2, eps = 0.5, 0.95, 0.0
    g = np.array([[3.0, -4.0, 0.0, 0.0]])
    theta, v, last = ob.rms_step_sparse(np.zeros((3, 4)), np.zeros(3), np.zeros(3, np.int64),
                                        np.array([1]), g, 1, eta, beta2, 0.0, eps)
    m = (9.0 + 16.0) / 4                           # mean squared gradient
    assert v[1] == pytest.approx((1 - beta2) * m, rel=1e-15)
    assert np.allclose(theta[1], -eta * g[0] / np.sqrt((1 - beta2) * m), rtol=1e-15)
    assert not theta[0].any() and not theta[2].any() and last.tolist() == [0, 1, 0]
    # pure decay of an untouched row over k steps
    th, vv, _ = ob.rms_flush(np.ones((1, 2)), np.array([2.0]), np.array([3]), 7, 0.1, 0.9, 0.5)
    assert np.allclose(th, (1 - 0.05) ** 4) and vv[0] == pytest.approx(2.0 * 0.9 ** 4)
