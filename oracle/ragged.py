"""Unpad-append-repad between ragged per-sequence caches and a left-padded
rectangle (oracle).  TEST INFRASTRUCTURE ONLY.

[Forensics] 3.2: EXSPEC keeps sequences in ragged states and batches
sequences of one length, which need no realignment; when no same-length group
forms it falls back to unpad-append-repad.  The ragged caches are one pool
[L][2][N][H][Cs][D] in which pool sequence s holds its n_s cached rows at
columns [0, n_s) of each (layer, K/V, head) plane; a batch is B distinct pool
sequences index[0..B) laid out as a rectangle [L][2][B][H][C][D].

These are the plain definitions, written as slice copies; cells outside the
copied ranges keep their contents.
"""
from __future__ import annotations

import numpy as np


def repad_kv(pool: np.ndarray, rect: np.ndarray, index, kv_len, E: int) -> np.ndarray:
    """Copy of `rect` in which member i holds pool sequence index[i]'s rows
    [0, kv_len[i]) at columns [E - kv_len[i], E) (left padding)."""
    out = rect.copy()
    for i, (s, n) in enumerate(zip(index, kv_len)):
        s, n = int(s), int(n)
        out[:, :, i, :, E - n:E, :] = pool[:, :, s, :, 0:n, :]
    return out


def unpad_kv(rect: np.ndarray, pool: np.ndarray, index, kv_len, emit_count, E: int) -> dict:
    """After the verify forward wrote k+1 slots at columns [E, E + k + 1) of
    the rectangle: each member keeps its cached rows and its first e_i slots
    (the last emitted token has no KV yet, [Forensics] App. D), i.e. columns
    [E - n_i, E + e_i), which are appended in order to its pool sequence's
    rows [0, n_i + e_i).  Returns the new pool and the new lengths."""
    out = pool.copy()
    new_len = []
    for i, (s, n, e) in enumerate(zip(index, kv_len, emit_count)):
        s, n, e = int(s), int(n), int(e)
        out[:, :, s, :, 0:n + e, :] = rect[:, :, i, :, E - n:E + e, :]
        new_len.append(n + e)
    return {"pool": out, "kv_len": np.array(new_len, np.int32)}


def ragged_bytes(kv_len, emit_count, col_bytes: int) -> dict:
    """Bytes read plus written by a repad (every cached row of every member)
    and by the following unpad (cached rows plus kept slots)."""
    n = np.asarray(kv_len, np.int64)
    e = np.asarray(emit_count, np.int64)
    return {"repad": int(2 * n.sum() * col_bytes), "unpad": int(2 * (n + e).sum() * col_bytes)}
