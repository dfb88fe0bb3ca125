"""Multi-round commit policies on a pool of sequences: EQSPEC against EXSPEC
(oracle).  TEST INFRASTRUCTURE ONLY.

[Forensics] 3.1: EQSPEC keeps each batch rectangular and realigns it after
every verification (unpad-append-repad, App. B).  [Forensics] 3.2: EXSPEC
keeps sequences ragged, forms batches of identical-length sequences from a
window larger than the batch (no realignment needed), and falls back to
unpad-append-repad for a batch that is not same-length.  [Forensics] 4.3 /
Table 5 compare the two by verification calls and alignment overhead.

Readings (the pages give the policies, not a loop):
  * a pool of N sequences; every round verifies every sequence exactly once,
    with inputs keyed by (sequence, round), so both policies emit the same
    tokens and differ only in batching and in the bytes they move;
  * EQSPEC: fixed batches of B consecutive sequences, each its own left-padded
    rectangle [L][2][B][H][C][D]; per batch and round: the verify forward
    writes k+1 slots at the rectangle's end column, one verify call, one
    realignment (commit_realign);
  * EXSPEC: the caches are one ragged pool [L][2][N][H][Cs][D] (sequence s at
    columns [0, n_s)); per round the window is the whole pool, grouped by
    group_same_length on the cached row counts n_s (equal exactly when the
    confirmed lengths are equal), batches of B, min_group; a
    same-length batch is verified with its slots written into the pool at
    [n_s, n_s + k + 1) and commits by a length update (commit_paged with one
    page per sequence: nothing moves); a mixed batch is repadded into a
    rectangle right-aligned at E = max n_s (repad_kv), verified with its slots
    at [E, E + k + 1), and unpadded back (unpad_kv);
  * greedy verification (greedy_verify) of planted drafts.
The verify forward's KV contents come from the caller (`forward`), standing
in for the target model.
"""
from __future__ import annotations

import numpy as np

from .greedy import greedy_verify
from .group import group_same_length
from .paged import commit_paged
from .ragged import ragged_bytes, repad_kv, unpad_kv
from .realign import commit_realign


def _slot_tokens(tokens, members, drafts) -> np.ndarray:
    """Tokens whose KV the forward writes into slots 0..k: the last confirmed
    token, then the drafts."""
    return np.array([[tokens[s][-1]] + [int(x) for x in drafts[s]] for s in members], np.int64)


def eqspec_round(st: dict, logits, drafts, dtype: str, k: int, forward) -> dict:
    """st: rects (list of [L,2,B,H,C,D] arrays), E (list), n [N], tokens (list
    of lists), B.  Updates st in place; returns the round's outputs."""
    B = st["B"]
    N = len(st["tokens"])
    emit = np.zeros(N, np.int32)
    out = np.full((N, k + 1), -1, np.int32)
    moved = 0
    for i, rect in enumerate(st["rects"]):
        m = np.arange(i * B, (i + 1) * B)
        E = st["E"][i]
        forward(rect, np.arange(B), m, np.full(B, E), st["n"][m], _slot_tokens(st["tokens"], m, drafts))
        v = greedy_verify(logits[m], dtype, drafts[m])
        c = commit_realign(rect, E, st["n"][m], v["emit_count"], k)
        st["rects"][i] = c["kv"]
        st["E"][i] = c["E_new"]
        st["n"][m] = c["kv_len"]
        moved += c["bytes_moved"]
        emit[m] = v["emit_count"]
        out[m] = v["out_tokens"]
        for j, s in enumerate(m):
            st["tokens"][s].extend(int(x) for x in v["out_tokens"][j][:v["emit_count"][j]])
    return dict(emit_count=emit, out_tokens=out, verify_calls=len(st["rects"]), bytes_moved=moved)


def exspec_round(st: dict, logits, drafts, dtype: str, k: int, forward) -> dict:
    """st: pool [L,2,N,H,Cs,D], rect [L,2,B,H,Cr,D] (the fallback buffer),
    n [N], tokens, B, min_group.  Updates st in place."""
    B, N = st["B"], len(st["tokens"])
    L, _, _, H, Cs, D = st["pool"].shape
    col_bytes = L * 2 * H * D * st["pool"].itemsize
    g = group_same_length(st["n"], B, st["min_group"])
    emit = np.zeros(N, np.int32)
    out = np.full((N, k + 1), -1, np.int32)
    moved = 0
    mixed = 0
    for t in range(g["num_batches"]):
        idx = g["perm"][g["batch_start"][t]:g["batch_start"][t + 1]].astype(np.int64)
        nb = len(idx)
        n_idx = st["n"][idx].copy()
        slots = _slot_tokens(st["tokens"], idx, drafts)
        v = greedy_verify(logits[idx], dtype, drafts[idx])
        if g["batch_len"][t] >= 0:
            forward(st["pool"], idx, idx, n_idx, n_idx, slots)
            pg = commit_paged(n_idx, v["emit_count"], k, Cs, idx[:, None].astype(np.int32))
            st["n"][idx] = pg["kv_len"]
        else:
            mixed += 1
            E = int(n_idx.max())
            st["rect"] = repad_kv(st["pool"], st["rect"], idx, n_idx, E)
            forward(st["rect"], np.arange(nb), idx, np.full(nb, E), n_idx, slots)
            u = unpad_kv(st["rect"], st["pool"], idx, n_idx, v["emit_count"], E)
            st["pool"] = u["pool"]
            st["n"][idx] = u["kv_len"]
            mb = ragged_bytes(n_idx, v["emit_count"], col_bytes)
            moved += mb["repad"] + mb["unpad"]
        emit[idx] = v["emit_count"]
        out[idx] = v["out_tokens"]
        for j, s in enumerate(idx):
            st["tokens"][s].extend(int(x) for x in v["out_tokens"][j][:v["emit_count"][j]])
    return dict(emit_count=emit, out_tokens=out, verify_calls=g["num_batches"], bytes_moved=moved,
                mixed_batches=mixed, grouping=g)
