"""CPU oracle of page staging from a host-resident table.

TEST INFRASTRUCTURE ONLY: imported by the tests and nothing on the product
path; shares no code with the HIP library.

Addresses are a pure function of the token IDs, known before the forward
pass, so the touched parts of a table kept in host memory can be fetched
ahead of the layer (PageGram §3.3; Engram notes §3.5). Readings where the
pages are silent:
  * "page" units: a PageGram page (K*S consecutive rows: the K heads of a
    token-order always share it); for the Engram-style tables a run of
    floor(4096 / row_bytes) rows of one per-head table, runs starting at the
    table's first row (the 4 KiB flash block of the page cache simulator;
    row_bytes counts NF4 as r/2 + 2). "row" units: single rows (what a
    device reading host memory at cache-line granularity can fetch);
  * a step stages each distinct unit its lookups touch once; the staged
    copy is bit-identical to the table, so e gathered from it equals e
    gathered from the table.
Pinned by tests/test_oracle_stage.py (PageGram: one unit per token-order;
Engram-style units equal the simulator's flash blocks; every row lies in
its unit; units partition the table).
"""
import numpy as np

from .pagesim import row_bytes

BLOCK = 4096


def unit_rows(lay, table_dtype, kind="page"):
    """Rows per staging unit."""
    if kind == "row":
        return 1
    if lay["kind"] == "pagegram":
        return lay["K"] * lay["S"]
    return max(1, BLOCK // row_bytes(table_dtype, lay["r"]))


def _head_tables(lay):
    O = lay["n_max"] - lay["n_min"] + 1
    sizes = [int(p) for p in lay["head_rows"][:O * lay["K"]]]
    bases = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    return bases, np.asarray(sizes, dtype=np.int64)


def units_of(lay, table_dtype, rows, kind="page"):
    """(first row, row count) of the unit holding each looked-up row;
    rows int [N, O, K]."""
    rows = np.asarray(rows, dtype=np.int64)
    if kind == "row":
        return rows.copy(), np.ones(rows.shape, dtype=np.int64)
    U = unit_rows(lay, table_dtype)
    if lay["kind"] == "pagegram":
        first = (rows // U) * U
        return first, np.full(rows.shape, U, dtype=np.int64)
    N, O, K = rows.shape
    bases, sizes = _head_tables(lay)
    hk = np.arange(O * K).reshape(O, K)
    base = bases[hk][None].repeat(N, 0)
    size = sizes[hk][None].repeat(N, 0)
    first = base + ((rows - base) // U) * U
    count = np.minimum(U, base + size - first)
    return first, count


def staged_units(lay, table_dtype, rows, kind="page"):
    """Distinct units of a step, ascending by first row: (first, count)."""
    first, count = units_of(lay, table_dtype, rows, kind)
    f, idx = np.unique(first.reshape(-1), return_index=True)
    return f, count.reshape(-1)[idx]


def staged_bytes(lay, table_dtype, rows, kind="page"):
    """Bytes moved from host memory for one step."""
    _, count = staged_units(lay, table_dtype, rows, kind)
    return int(count.sum()) * row_bytes(table_dtype, lay["r"])
