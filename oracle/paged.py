"""Commit for a variable-length (paged) KV layout: rollback only (oracle).
TEST INFRASTRUCTURE ONLY.

[Forensics] section 2 and App. F: variable-length layouts pack each sequence
separately, so no rectangle has to be restored after a verify round, but the
rejected tokens must still be rolled back in both the position ids and the KV
cache.  With a paged cache (fixed-size pages listed per sequence in a block
table) the plain definition is:

  before the verify forward, sequence b held n_b cached rows; the caller gave
  it pages for the forward's k + 1 slots, so its first
  a_b = ceil((n_b + k + 1) / page) block-table entries are in use;
  after verification it keeps e_b slots ([Forensics] App. D: the last emitted
  token has no KV yet), so n'_b = n_b + e_b rows and ceil(n'_b / page) pages;
  the next input position is n'_b;
  the block-table entries ceil(n'_b / page) .. a_b - 1 are released, listed
  in block-table order, sequences in batch order, with their offsets as an
  exclusive prefix sum;
  nothing moves: rows of rejected slots that share a kept page stay as stale
  bytes past n'_b.
Invalid sequences (n_b < 0, e_b outside [0, k + 1], a_b beyond the block
table's width) get status bits, keep n_b, and release nothing.
"""
from __future__ import annotations

import numpy as np

from .status import ST_BAD_STATE, ST_CAPACITY


def pages_for(rows: int, page: int) -> int:
    return -(-int(rows) // int(page))


def commit_paged(n, e, k: int, page: int, block_table) -> dict:
    """n, e: [B]; block_table: [B, max_pages] int32 page ids."""
    bt = np.asarray(block_table)
    B, max_pages = bt.shape
    kv_len = np.zeros(B, np.int32)
    pages_kept = np.zeros(B, np.int32)
    status = np.zeros(B, np.int32)
    freed = []
    offsets = [0]
    for b in range(B):
        nb, eb = int(n[b]), int(e[b])
        st = 0
        if nb < 0 or eb < 0 or eb > k + 1:
            st |= ST_BAD_STATE
        elif pages_for(nb + k + 1, page) > max_pages:
            st |= ST_CAPACITY
        if st:
            status[b] = st
            kv_len[b] = nb
            pages_kept[b] = pages_for(max(nb, 0), page)
            offsets.append(len(freed))
            continue
        new_len = nb + eb
        used = pages_for(nb + k + 1, page)
        keep = pages_for(new_len, page)
        kv_len[b] = new_len
        pages_kept[b] = keep
        freed.extend(int(x) for x in bt[b, keep:used])
        offsets.append(len(freed))
    return dict(kv_len=kv_len, pages_kept=pages_kept, freed=np.array(freed, np.int32),
                freed_offsets=np.array(offsets, np.int32), status=status, bytes_moved=0)


def gather_rows(pool, block_table, b: int, rows: int, page: int):
    """Rows 0..rows-1 of sequence b read through its block table.

    pool: [num_pages, page, ...]; returns [rows, ...]."""
    idx = np.arange(rows)
    return pool[np.asarray(block_table)[b, idx // page], idx % page]


def write_rows(pool, block_table, b: int, positions, values, page: int) -> None:
    """Store values[i] at row positions[i] of sequence b (through its block table)."""
    pos = np.asarray(positions)
    pool[np.asarray(block_table)[b, pos // page], pos % page] = values
