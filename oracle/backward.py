"""CPU oracle of the backward pass and the sparse table update.

TEST INFRASTRUCTURE ONLY: imported by the tests and nothing on the product
path; shares no code with the HIP library. Plain numpy, float64.

The scalar-gated forward out = x + g W_V e (PageGram §2.2, §3.1) has
  dL/dx  = dy
  dL/dW  = g dy^T e                       (dW_V, [d x E])
  dL/de  = g dy W                         ([N x E])
and, since e_t is the concatenation of s_{t,n,k} (.) T[row_{t,n,k}], the table
gradient is non-zero only on touched rows:
  dL/dT[row] = sum over lookups (t, n, k) with row_{t,n,k} = row of
               s_{t,n,k} (.) dL/de_t[(n, k) slice]
(the "sparse gradient"; PageGram §9.4 check 4 requires it to equal the dense
table gradient).

Table optimiser (PageGram §3.3 and §9.1): tables start at zero; every row
keeps a moving average v of its squared gradient (beta2 = 0.95); a step
moves the row by eta g / sqrt(v); steps in which a row is not touched are
applied later as replayed decay (§3.3), so the lazy per-row update equals
the dense one that visits every row every step with a zero gradient.
Readings where the pages are silent:
  * "row-wise": v is one scalar per row, the moving average of the row's
    mean squared gradient;
  * no bias correction (none is mentioned);
  * the step divides by sqrt(v) + eps (eps a parameter) and applies
    decoupled weight decay lambda (a parameter; the pages give no value):
        theta <- theta (1 - eta lambda) - eta g / (sqrt(v) + eps);
  * a row touched at step t after last at step tau first replays the
    skipped steps tau+1..t-1 (theta scaled by (1 - eta lambda)^(t-tau-1);
    v scaled by beta2^(t-tau-1) together with the beta2 of step t).
Parity: pinned by a finite-difference check of dW and de, the dense table
gradient (check 4), the dense optimiser run, and closed forms of one step
(tests/test_oracle_backward.py).
"""
import numpy as np


def backward_dense(e, W, g, dy):
    """dW = g dy^T e and de = g dy W (float64)."""
    e = np.asarray(e, np.float64)
    W = np.asarray(W, np.float64)
    dy = np.asarray(dy, np.float64)
    return g * (dy.T @ e), g * (dy @ W)


def row_gradients(layout, rows, signs, de):
    """Sparse table gradient: (urows ascending, grads [len(urows), r]).

    rows int [N, O, K], signs uint64 [N, O, K, ceil(r/64)], de [N, O*K*r].
    Each row's gradient is summed over its lookups in lookup order
    (t, then n, then k)."""
    from .pagegram import sign_vectors
    r = layout["r"]
    rows = np.asarray(rows, np.int64)
    N, O, K = rows.shape
    de = np.asarray(de, np.float64).reshape(N, O, K, r)
    if layout["use_signs"]:
        de = de * sign_vectors(signs, r)
    flat_rows = rows.reshape(-1)
    flat_g = de.reshape(-1, r)
    urows = np.unique(flat_rows)
    pos = {int(u): i for i, u in enumerate(urows)}
    grads = np.zeros((len(urows), r), np.float64)
    for q in range(len(flat_rows)):            # lookup order
        grads[pos[int(flat_rows[q])]] += flat_g[q]
    return urows, grads


def dense_table_gradient(layout, n_rows, rows, signs, de):
    """The same gradient as a dense [n_rows, r] array (every table row)."""
    from .pagegram import sign_vectors
    r = layout["r"]
    rows = np.asarray(rows, np.int64)
    N, O, K = rows.shape
    de = np.asarray(de, np.float64).reshape(N, O, K, r)
    if layout["use_signs"]:
        de = de * sign_vectors(signs, r)
    G = np.zeros((n_rows, r), np.float64)
    np.add.at(G, rows.reshape(-1), de.reshape(-1, r))
    return G


def rms_step_dense(theta, v, G, eta, beta2, lam, eps):
    """One optimiser step on every row (G = 0 for untouched rows)."""
    theta = np.asarray(theta, np.float64)
    G = np.asarray(G, np.float64)
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * np.mean(G * G, axis=1)
    theta = theta * (1.0 - eta * lam) - eta * G / (np.sqrt(v) + eps)[:, None]
    return theta, v


def rms_step_sparse(theta, v, last, urows, grads, step, eta, beta2, lam, eps):
    """One lazy step at `step` on the touched rows only (copies returned).
    last[row] is the step of the row's previous update (its state is current
    as of that step)."""
    theta = np.array(theta, np.float64)
    v = np.array(v, np.float64)
    last = np.array(last, np.int64)
    for u, g in zip(np.asarray(urows, np.int64), np.asarray(grads, np.float64)):
        skipped = step - int(last[u]) - 1
        decay = (1.0 - eta * lam) ** skipped
        vv = (beta2 ** (skipped + 1)) * v[u] + (1.0 - beta2) * np.mean(g * g)
        theta[u] = theta[u] * decay * (1.0 - eta * lam) - eta * g / (np.sqrt(vv) + eps)
        v[u] = vv
        last[u] = step
    return theta, v, last


def rms_flush(theta, v, last, step, eta, beta2, lam):
    """Bring every row to `step` (replay the decay of its untouched steps)."""
    theta = np.array(theta, np.float64)
    v = np.array(v, np.float64)
    last = np.array(last, np.int64)
    k = (step - last).astype(np.float64)
    theta = theta * ((1.0 - eta * lam) ** k)[:, None]
    v = v * beta2 ** k
    last[:] = step
    return theta, v, last
