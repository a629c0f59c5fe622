"""Pins of the flash page-cache oracle (oracle/pagesim.py) and parity of the
library's host simulator (pg_flash_blocks, pg_lru_cache_sim) with it.

What pins the oracle, independently of its own code:
  * the pages' exact uncached counts: a PageGram token touches exactly one
    block per order (2 reads), an Engram-style token one block per head
    (16 reads) -- PageGram §2.3, Fig. 2, §8;
  * the pages' NF4 storage arithmetic (34-byte rows, 120 per 4 KiB block,
    three 1,088-byte pages per block at S = 4) -- PageGram §2.3, §3.3;
  * LRU closed forms: no cache -> every distinct block is a read; a cache
    holding everything -> only compulsory misses; a cyclic stream over C + 1
    blocks with C slots misses every time; LRU is a stack algorithm, so misses
    never grow with capacity (Mattson et al. 1970);
  * an independent list-based LRU on random small streams.
"""
import numpy as np
import pytest

import oracle
from oracle import pagesim
from synth import configs
import synth


def _idx(wl, n_tok):
    toks = synth.tokens(wl)[:, :n_tok] if wl["T"] >= n_tok else synth.tokens(wl)
    return oracle.index(wl["layout"], toks[:1], synth.canon_map(wl), wl["canon_vocab"])


def test_nf4_storage_arithmetic():
    assert pagesim.row_bytes("nf4", 64) == 34
    assert pagesim.BLOCK // pagesim.row_bytes("nf4", 64) == 120
    # S = 4: 8 * 4 * 34 = 1088-byte pages, three per block
    lay = configs.workload(3)["layout"]
    page = lay["K"] * lay["S"] * pagesim.row_bytes("nf4", 64)
    assert page == 1088 and pagesim.BLOCK // page == 3
    rows = np.arange(0, 6 * 32, 32, dtype=np.int64)         # first row of pages 0..5
    assert pagesim.flash_blocks(lay, "nf4", rows).tolist() == [0, 0, 0, 1, 1, 1]


@pytest.mark.parametrize("i", [3, 5])
def test_pagegram_touches_one_block_per_order(i):
    wl = configs.workload(i)
    lay = wl["layout"]
    ref = _idx(wl, 1500)
    blocks = pagesim.flash_blocks(lay, "nf4", ref["rows"])      # [T, O, K]
    per_tok = [len(s) for s in pagesim.token_blocks(blocks.reshape(len(blocks), -1))]
    # every head of a token-order lies in one page, pages of different orders
    # never share a block (P_2 is a multiple of the pages per block)
    assert set(per_tok) == {2}
    st = pagesim.lru_simulate(blocks.reshape(len(blocks), -1), 0)
    assert st["misses"] == st["distinct"] == 2 * len(blocks)


def test_engram_touches_one_block_per_head():
    wl = configs.workload(2)                        # Engram-style prime tables
    lay = wl["layout"]
    ref = _idx(wl, 1500)
    blocks = pagesim.flash_blocks(lay, "nf4", ref["rows"])
    per_tok = [len(s) for s in pagesim.token_blocks(blocks.reshape(len(blocks), -1))]
    assert set(per_tok) == {16}                     # each head table is its own region


def test_lru_closed_forms():
    rng = np.random.default_rng(7)
    blocks = rng.integers(0, 50, size=(400, 4))
    n_distinct = len(np.unique(blocks))
    none = pagesim.lru_simulate(blocks, 0)
    allc = pagesim.lru_simulate(blocks, 50)
    assert none["misses"] == none["distinct"]
    assert allc["misses"] == n_distinct
    # cyclic stream over C + 1 blocks, one block per token
    C = 7
    cyc = np.tile(np.arange(C + 1), 20).reshape(-1, 1)
    assert pagesim.lru_simulate(cyc, C)["misses"] == len(cyc)
    assert pagesim.lru_simulate(cyc, C + 1)["misses"] == C + 1
    # stack property: misses never increase with capacity
    m = [pagesim.lru_simulate(blocks, c)["misses"] for c in range(0, 52, 3)]
    assert all(a >= b for a, b in zip(m, m[1:]))


def _lru_list(blocks, cap):
    """Independent LRU: a Python list, most recent last."""
    cache, misses = [], 0
    for row in blocks:
        for b in dict.fromkeys(int(x) for x in row):
            if b in cache:
                cache.remove(b)
                cache.append(b)
            else:
                misses += 1
                if cap > 0:
                    cache.append(b)
                    if len(cache) > cap:
                        cache.pop(0)
    return misses


def test_lru_matches_list_model():
    rng = np.random.default_rng(11)
    for trial in range(20):
        blocks = rng.integers(0, 30, size=(120, 3))
        cap = int(rng.integers(0, 25))
        assert pagesim.lru_simulate(blocks, cap)["misses"] == _lru_list(blocks, cap)


# ----------------------------------------------------------------------------
# The library's host simulator against the oracle (no GPU needed)


@pytest.mark.parametrize("i", [1, 2, 3, 5])
def test_library_flash_blocks_match_oracle(i):
    import hashed_head_gram_amd as pg
    from tests.gpu_inputs import layout_of
    wl = configs.workload(i)
    ref = _idx(wl, 800)
    want = pagesim.flash_blocks(wl["layout"], wl["table_dtype"], ref["rows"])
    dt = {"f32": pg.PG_F32, "bf16": pg.PG_BF16, "nf4": pg.PG_NF4}[wl["table_dtype"]]
    got = pg.pg_flash_blocks(layout_of(wl), dt, ref["rows"].astype(np.int64))
    assert np.array_equal(got, want)


def test_library_lru_matches_oracle():
    import hashed_head_gram_amd as pg
    rng = np.random.default_rng(3)
    # Zipf-like reuse: a few hot blocks and a long tail
    hot = rng.integers(0, 40, size=(3000, 16))
    tail = rng.integers(0, 20000, size=(3000, 16))
    blocks = np.where(rng.random((3000, 16)) < 0.6, hot, tail).astype(np.int64)
    for cap in (0, 1, 17, 500, 4096, 60000):
        want = pagesim.lru_simulate(blocks, cap)
        got = pg.pg_lru_cache_sim(blocks, cap)
        assert got == want, (cap, got, want)


def test_library_simulator_rejects_bad_arguments():
    import hashed_head_gram_amd as pg
    from tests.gpu_inputs import layout_of
    wl = configs.workload(3)
    with pytest.raises(pg.PagegramError):
        pg.pg_flash_blocks(layout_of(wl), pg.PG_NF4, np.array([-1], dtype=np.int64))
    with pytest.raises(pg.PagegramError):
        pg.pg_lru_cache_sim(np.zeros((2, 2), dtype=np.int64), -1)
