"""Commit and realignment of the left-padded KV rectangle (oracle).
TEST INFRASTRUCTURE ONLY.

What the step must restore ([Forensics] section 3 / 3.1 and App. B): after a
verify round the batch must again be a rectangle whose sequences are all
right-aligned to one end column (rectangular alignment), each sequence's
position ids must run 0, 1, 2, ... over its cells (position-id contiguity),
and every kept KV cell must hold the target-computed entry of the token at
that position (position / KV-cache correspondence).  Realignment keeps the
retained entries, drops the entries of rejected drafts, keeps the target's
values for accepted tokens, and rebuilds position ids from the attention mask
after re-padding.  Under uniform acceptance (or one sequence) the padding is
unchanged and nothing moves (App. B).

Which new slots survive ([Forensics] App. D; [Walkthrough] 5.2): the verify
forward wrote k+1 slots per sequence (the last confirmed token, then the
drafts).  A sequence that emitted e tokens keeps the first e slots; its last
emitted token (correction, bonus or EOS) has no KV until the next forward.

Plain definition used here -- unpad, append, repad, never in place:
  n'_b = n_b + e_b, M = max_b e_b, E' = E + M;
  take sequence b's cells at columns [E - n_b, E + e_b) of every (layer, K/V,
  head) plane and write them, in order, to columns [E' - n'_b, E') of a copy
  of the old buffer.
  mask[b, c] = 1 exactly for c in [E' - n'_b, E'), over all C columns;
  pos[b, c] = (running count of mask[b, 0..c]) - 1 where the mask is 1, else 0.
  bytes_moved = sum over sequences that shift (M - e_b > 0) of
                2 * n'_b * (bytes of one column across all planes).
Inputs that break the preconditions (E < 0, E + k + 1 > C, n_b outside
[0, E], e_b outside [0, k + 1]) produce status bits and no other output.
"""
from __future__ import annotations

import numpy as np

from .status import ST_BAD_STATE, ST_CAPACITY


def commit_bookkeeping(E: int, n, e, k: int, C: int) -> dict:
    n = [int(x) for x in n]
    e = [int(x) for x in e]
    B = len(n)
    status = np.zeros(B, np.int32)
    if E < 0 or E + k + 1 > C:
        status[:] = ST_CAPACITY
    for b in range(B):
        if n[b] < 0 or n[b] > E or e[b] < 0 or e[b] > k + 1:
            status[b] |= ST_BAD_STATE
    if status.any():
        return dict(ok=False, status=status)
    M = max(e) if B else 0
    return dict(ok=True, status=status, M=M, E_new=E + M,
                n_new=np.array([n[b] + e[b] for b in range(B)], np.int64),
                delta=np.array([M - e[b] for b in range(B)], np.int64))


def position_and_mask(E_new: int, n_new, C: int):
    B = len(n_new)
    mask = np.zeros((B, C), np.int32)
    pos = np.zeros((B, C), np.int32)
    for b in range(B):
        mask[b, E_new - int(n_new[b]):E_new] = 1
        running = np.cumsum(mask[b]) - 1
        pos[b] = np.where(mask[b] == 1, running, 0)
    return pos, mask


def commit_realign(kv, E: int, n, e, k: int, C: int | None = None) -> dict:
    """kv: None (bookkeeping only) or an array [L, 2, B, H, C, D] of element bits."""
    if C is None:
        C = kv.shape[4]
    book = commit_bookkeeping(E, n, e, k, C)
    if not book["ok"]:
        return book
    n = np.asarray(n, np.int64)
    e = np.asarray(e, np.int64)
    E_new, n_new, delta = book["E_new"], book["n_new"], book["delta"]
    pos, mask = position_and_mask(E_new, n_new, C)
    out = dict(book, pos=pos, mask=mask, kv_len=n_new)
    if kv is not None:
        L, _, B, H, _, D = kv.shape
        col_bytes = L * 2 * H * D * kv.itemsize
        new = kv.copy()
        for b in range(B):
            src = kv[:, :, b, :, E - n[b]:E + e[b], :]           # unpad + append
            new[:, :, b, :, E_new - n_new[b]:E_new, :] = src      # repad (right-aligned at E')
        out["kv"] = new
        out["bytes_moved"] = int(sum(2 * int(n_new[b]) * col_bytes
                                     for b in range(B) if delta[b] > 0))
    return out


def moved_bytes(n_new, delta, col_bytes: int) -> int:
    """bytes_moved without touching the cache (for shapes too large to copy on the host)."""
    return int(sum(2 * int(n_new[b]) * col_bytes for b in range(len(n_new)) if delta[b] > 0))


def resync_draft(kv, E: int, n, e, k: int, C: int | None = None) -> dict:
    """Re-sync of the draft model's KV rectangle to the accepted prefix.

    [Design] "KV Cache Synchronization" and step 7 of the Standard Greedy
    Algorithm: after each step the draft cache must hold the accepted prefix,
    copying the accepted entries rather than re-running the draft.  An
    autoregressive draft that proposed d_1..d_k consumed the last confirmed
    token and d_1..d_{k-1}, so its forward wrote k slots [E, E + k), one fewer
    than the verify forward.  A sequence that emitted e tokens keeps the first
    min(e, k) of them; after full acceptance (e = k + 1) the draft holds no KV
    for d_k yet and is one entry behind the target.  Realignment is then the
    unpad-append-repad of commit_realign with min(e, k) in place of e:
    n'_b = n_b + min(e_b, k), E' = E + max_b min(e_b, k).
    Preconditions: E + k <= C, n_b in [0, E], e_b in [0, k + 1].
    """
    if C is None:
        C = kv.shape[4]
    e = [int(x) for x in e]
    n = [int(x) for x in n]
    B = len(n)
    status = np.zeros(B, np.int32)
    if E < 0 or E + k > C:
        status[:] = ST_CAPACITY
    for b in range(B):
        if n[b] < 0 or n[b] > E or e[b] < 0 or e[b] > k + 1:
            status[b] |= ST_BAD_STATE
    if status.any():
        return dict(ok=False, status=status)
    kept = [min(x, k) for x in e]
    # the same repad with k - 1 in the role of k: k + 1 - 1 = k slots written
    out = commit_realign(kv, E, n, kept, k - 1, C)
    out["kept"] = np.array(kept, np.int64)
    return out
