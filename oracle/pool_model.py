"""Byte-level model of the paged K/V pool (oracle; test infrastructure only).

The pages describe K and V as pools of fixed-size pages, each logical page of a
sequence mapped to a pool page through an int32 block table, one row per
position (llama.cpp-PR2, page-table commit: K/V are a pool of pages;
KV-streaming commit: per-layer page tables are one I32 input).  The pages do
not fix how rows are laid out inside a pool page.  The reading taken here:

* K and V are separate pools (``pa_decode`` takes ``k_pool`` and ``v_pool``);
* a pool is ``[n_blocks][n_kv_heads][page_size][row_bytes]`` bytes
  (head-major inside a page, so one KV head's rows of one page are
  contiguous);
* a sequence's position ``pos`` lives in logical page ``pos // page_size``
  at slot ``pos % page_size``.

Two operations are modelled: the append scatter (rows into (page, slot)
destinations) and the logical gather through a block-table row.  Both are
written independently of the HIP library.
"""

import numpy as np


def scatter_rows(pool: np.ndarray, blocks, slots, rows: np.ndarray) -> np.ndarray:
    """Append model (colibri#372, Summary: only the new rows are uploaded and a
    scatter puts them into pages).  ``rows`` is ``[n][n_kv_heads][row_bytes]``;
    row i goes to page ``blocks[i]``, slot ``slots[i]``, for every KV head.
    Rows are written in order, so when two rows name the same destination the
    later one is kept.  Returns a new pool; the input pool is not modified.
    An out-of-range destination raises ``IndexError`` before anything is
    written."""
    out = pool.copy()
    n_blocks, n_kv_heads, page_size, rb = out.shape
    rows = np.asarray(rows, dtype=np.uint8)
    if rows.ndim != 3 or rows.shape[1:] != (n_kv_heads, rb):
        raise ValueError("rows must be [n][n_kv_heads][row_bytes]")
    for i in range(rows.shape[0]):
        b, s = int(blocks[i]), int(slots[i])
        if not (0 <= b < n_blocks and 0 <= s < page_size):
            raise IndexError(f"row {i}: destination (block {b}, slot {s}) out of range")
    for i in range(rows.shape[0]):
        b, s = int(blocks[i]), int(slots[i])
        for h in range(n_kv_heads):
            out[b, h, s, :] = rows[i, h, :]
    return out


def gather_rows(pool: np.ndarray, table_row, seq_len: int) -> np.ndarray:
    """Logical rows ``[n_kv_heads][seq_len][row_bytes]`` of one sequence, read
    page by page through its block-table row (llama.cpp-PR2, page-table
    commit: the CPU path gathers the logical rows into a work buffer).
    Raises ``IndexError`` for a table entry outside the pool or a table row too
    short for ``seq_len``."""
    n_blocks, n_kv_heads, page_size, rb = pool.shape
    out = np.empty((n_kv_heads, seq_len, rb), dtype=np.uint8)
    table_row = np.asarray(table_row)
    # Logical page lp holds positions [lp*P, lp*P + P): slot = pos - lp*P.
    for lp in range(-(-seq_len // page_size)):
        if lp >= table_row.shape[0]:
            raise IndexError(f"position {lp * page_size} needs table entry {lp}, row has {table_row.shape[0]}")
        b = int(table_row[lp])
        if not (0 <= b < n_blocks):
            raise IndexError(f"table entry {lp} = {b} outside a pool of {n_blocks} pages")
        first = lp * page_size
        n = min(page_size, seq_len - first)
        out[:, first:first + n, :] = pool[b, :, 0:n, :]
    return out
