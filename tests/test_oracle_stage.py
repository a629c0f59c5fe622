"""Pins of the page-staging oracle (oracle/stage.py).

Independent of its own formulas:
  * PageGram: every token-order's K rows share one unit, so a token stages
    at most 2 units, and the unit is the page of the row formula
    (PageGram §3.1: K*S rows per page);
  * Engram-style units are exactly the 4 KiB flash blocks of the page-cache
    oracle (a separate implementation, oracle/pagesim.py);
  * every looked-up row lies inside its unit, units never straddle a
    per-head table, and the units of all rows partition the table.
"""
import numpy as np
import pytest

import oracle
from oracle import pagesim, stage
from synth import configs
import synth


def _rows(wl, n_tok=600):
    toks = synth.tokens(wl)[:1, :n_tok]
    return oracle.index(wl["layout"], toks, synth.canon_map(wl), wl["canon_vocab"])["rows"]


@pytest.mark.parametrize("i", [1, 3, 5])
def test_pagegram_one_unit_per_token_order(i):
    wl = configs.workload(i)
    lay = wl["layout"]
    rows = _rows(wl)
    first, count = stage.units_of(lay, wl["table_dtype"], rows)
    assert (first == first[:, :, :1]).all()                  # K heads share the unit
    pages = rows // (lay["K"] * lay["S"])
    assert np.array_equal(first, pages * lay["K"] * lay["S"])
    assert (count == lay["K"] * lay["S"]).all()
    f, c = stage.staged_units(lay, wl["table_dtype"], rows)
    assert len(f) <= 2 * rows.shape[0]


@pytest.mark.parametrize("i,dt", [(2, "bf16"), (6, "nf4")])
def test_engram_units_are_flash_blocks(i, dt):
    wl = configs.workload(i)
    lay = wl["layout"]
    rows = _rows(wl)
    first, count = stage.units_of(lay, dt, rows)
    blocks = pagesim.flash_blocks(lay, dt, rows)
    # same partition: equal blocks <=> equal units
    fb = {}
    for f, b in zip(first.reshape(-1), blocks.reshape(-1)):
        assert fb.setdefault(int(b), int(f)) == int(f)
    assert len(set(fb.values())) == len(fb)
    assert np.all(rows >= first) and np.all(rows < first + count)


def test_units_partition_a_small_table():
    lay = dict(kind="engram", n_min=2, n_max=3, K=2, S=1, r=64, pages=[],
               head_rows=[70, 33, 129, 5], hash_seed=1, use_signs=1)
    R = 70 + 33 + 129 + 5
    rows = np.arange(R).reshape(-1, 1, 1)
    # put every row in the head slot of the table it belongs to
    bases = [0, 70, 103, 232]
    hk = np.searchsorted(bases, np.arange(R), side="right") - 1
    full = np.zeros((R, 2, 2), dtype=np.int64)
    for q in range(R):
        full[q, hk[q] // 2, hk[q] % 2] = q
        for h in range(4):
            if h != hk[q]:
                full[q, h // 2, h % 2] = bases[h]      # a valid row of head h
    first, count = stage.units_of(lay, "bf16", full)
    U = stage.unit_rows(lay, "bf16")
    assert U == 32
    f = first[np.arange(R), hk // 2, hk % 2]
    c = count[np.arange(R), hk // 2, hk % 2]
    # each table is cut into runs of 32 from its own first row
    for h, (b, n) in enumerate(zip(bases, [70, 33, 129, 5])):
        sel = hk == h
        assert np.array_equal(f[sel], b + (np.arange(n) // 32) * 32)
        assert np.all(c[sel] == np.minimum(32, b + n - f[sel]))
    # the distinct units cover every row exactly once
    uf, uc = np.unique(f, return_index=True)
    assert int(c[uc].sum()) == R
    assert stage.staged_bytes(lay, "bf16", full[:, :, :]) >= R * 128


@pytest.mark.parametrize("i", [1, 2])
def test_row_units_are_the_distinct_rows(i):
    wl = configs.workload(i)
    rows = _rows(wl)
    f, c = stage.staged_units(wl["layout"], wl["table_dtype"], rows, kind="row")
    assert np.array_equal(f, np.unique(rows)) and (c == 1).all()
    assert stage.staged_bytes(wl["layout"], wl["table_dtype"], rows, kind="row") == \
        len(np.unique(rows)) * 2 * wl["layout"]["r"]

