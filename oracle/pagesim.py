"""CPU oracle of the flash page-cache simulation (page-touch trace + LRU).

TEST INFRASTRUCTURE ONLY: imported by the tests and nothing on the product
path; shares no code with the library's C++ simulator.

What it models (PageGram tech report §2.3, §3.3, §8 Fig. 4a and appendix D):
a table stored on flash is read in 4 KiB blocks; each token looks up 2K head
rows (K heads for each of the two n-gram orders); a RAM page cache with LRU
replacement holds whole blocks, and every lookup whose block is not cached
costs one random flash read. A token reads each distinct block it needs once.

Storage order (the pages' layouts):
  * PageGram: a page is K*S consecutive head rows. If a page fits in a block,
    floor(4096 / page_bytes) whole pages share a block (PG §3.3: three
    1,088-byte NF4 pages per block at S = 4, one 4,080-byte page at S = 15);
    otherwise a page spans ceil(page_bytes / 4096) blocks and a row falls in
    the block of its byte offset inside the page.
  * Engram-style: each per-head table is its own file region, rows packed
    floor(4096 / row_bytes) per block (120 NF4 rows of 34 bytes, PG §2.3),
    every table starting on a fresh block.

Readings: blocks of different orders' pages are numbered in one global page
sequence (orders in ascending n); a token's blocks are offered to the cache in
(order, head) order, duplicates within the token dropped. Parity of the
absolute reads/token with the report's 20M-token test set is unpinned (the
set is not here); the exact counts pinned are the uncached ones (2 vs up to
16) and the LRU closed forms in tests/test_oracle_pagesim.py.
"""
from collections import OrderedDict

import numpy as np

BLOCK = 4096


def row_bytes(table_dtype, r):
    """Stored bytes of one head row: fp32 4r, bf16 2r, NF4 r/2 codes + fp16 scale."""
    return {"f32": 4 * r, "bf16": 2 * r, "nf4": r // 2 + 2}[table_dtype]


def flash_blocks(lay, table_dtype, rows):
    """4 KiB block index of every looked-up row; rows int [..., K] (any
    leading shape, as pg_index writes them). Returns int64 of the same shape."""
    rows = np.asarray(rows, dtype=np.int64)
    rb = row_bytes(table_dtype, lay["r"])
    K = lay["K"]
    if lay["kind"] == "pagegram":
        S = lay["S"]
        page_bytes = K * S * rb
        page = rows // (K * S)                      # global page number
        if page_bytes <= BLOCK:
            return page // (BLOCK // page_bytes)
        per_page = -(-page_bytes // BLOCK)
        return page * per_page + ((rows % (K * S)) * rb) // BLOCK
    # Engram-style: per-head tables, each starting on a fresh block.
    rpb = BLOCK // rb
    n_heads = (lay["n_max"] - lay["n_min"] + 1) * K
    sizes = [int(p) for p in lay["head_rows"][:n_heads]]   # (order, head) order
    row_base, blk_base = [], []
    acc_r = acc_b = 0
    for p in sizes:
        row_base.append(acc_r)
        blk_base.append(acc_b)
        acc_r += p
        acc_b += -(-p // rpb)
    row_base = np.array(row_base, dtype=np.int64)
    blk_base = np.array(blk_base, dtype=np.int64)
    t = np.searchsorted(row_base, rows, side="right") - 1   # which head table
    return blk_base[t] + (rows - row_base[t]) // rpb


def token_blocks(blocks):
    """Per token, its distinct blocks in first-use order; blocks [n_tok, L]."""
    out = []
    for row in np.asarray(blocks, dtype=np.int64).reshape(len(blocks), -1):
        seen = []
        for b in row.tolist():
            if b not in seen:
                seen.append(b)
        out.append(seen)
    return out


def lru_simulate(blocks, capacity):
    """Offer each token's distinct blocks to an LRU cache of `capacity`
    blocks. Returns dict(tokens, lookups, distinct, misses): lookups = row
    lookups, distinct = sum of distinct blocks per token (the uncached reads),
    misses = flash reads."""
    blocks = np.asarray(blocks, dtype=np.int64)
    n = len(blocks)
    cache = OrderedDict()
    misses = distinct = 0
    for seen in token_blocks(blocks):
        distinct += len(seen)
        for b in seen:
            if b in cache:
                cache.move_to_end(b)
                continue
            misses += 1
            if capacity <= 0:
                continue
            cache[b] = True
            if len(cache) > capacity:
                cache.popitem(last=False)
    return dict(tokens=n, lookups=int(blocks.size), distinct=distinct, misses=misses)
