"""Greedy verification of a candidate tree, and compaction of the accepted
path's KV slots (oracle).  TEST INFRASTRUCTURE ONLY.

The pages name tree-structured verification ([Forensics] section 5) and the
fields a tree verifier records ([Walkthrough] 5.2: draft tokens, positions, a
visibility mask and retrieve_* indices) but give no algorithm.  Reading used
here, the plain greedy rule of [Walkthrough] 4.1 applied along a tree:

  each sequence has a tree of N nodes in topological order (a parent's index
  is below its children's); node 0 is the root, standing for the last
  confirmed token; node i > 0 proposes token draft[b, i];
  first_child[b, i] / next_sibling[b, i] (-1 = none) list each node's children
  in order (the retrieve-next-token / retrieve-next-sibling links);
  the target forward over the tree gives one logit row per node: row i is the
  distribution of the token after the path ending at node i;
  verification starts at the root: t = argmax(row of the current node) (lowest
  index on ties); the first child (in sibling order) proposing t is accepted
  and becomes the current node; otherwise t is emitted as the correction (or,
  at a leaf, the bonus) and the round stops.  EOS and the budget stop it as in
  the linear case;
  the forward wrote one KV slot per node at columns E + i; the kept slots are
  the root and the accepted nodes (e_b of them: the last emitted token has no
  KV yet), moved in path order to columns E .. E + e_b - 1 so that the
  sequence's rows are contiguous again; the rectangle is then realigned as in
  the linear commit.

A linear chain (node i's only child is node i + 1) reduces exactly to the
greedy verification of a k-token draft.
"""
from __future__ import annotations

import numpy as np

from .greedy import argmax_first, widen_bf16
from .status import ST_DRAFT_OOR, ST_BAD_STATE


def tree_verify(logits: np.ndarray, dtype: str, draft, first_child, next_sibling,
                eos_id: int = -1, remaining=None) -> dict:
    """logits [B, N, V] (f32 values or bf16 bits); draft, first_child,
    next_sibling [B, N] int.  Returns accept_len, emit_count, out_tokens
    [B, N] (-1 padded), path [B, N] (kept node indices in order, -1 padded),
    emit_offsets [B+1], status [B]."""
    x = widen_bf16(logits) if dtype == "bf16" else np.asarray(logits, np.float32)
    B, N, V = x.shape
    eos = None if eos_id < 0 else int(eos_id)
    accept_len = np.zeros(B, np.int32)
    emit_count = np.zeros(B, np.int32)
    out_tokens = np.full((B, N), -1, np.int32)
    path = np.full((B, N), -1, np.int32)
    status = np.zeros(B, np.int32)
    for b in range(B):
        st = 0
        for i in range(1, N):
            if not 0 <= int(draft[b, i]) < V:
                st |= ST_DRAFT_OOR
        ok = True
        for i in range(N):                       # links must point forward and stay inside the tree
            for link in (int(first_child[b, i]), int(next_sibling[b, i])):
                if link != -1 and not (i < link < N):
                    ok = False
        if not ok:
            status[b] = st | ST_BAD_STATE
            continue
        rem = None if remaining is None else int(remaining[b])
        out, nodes, acc = [], [0], 0
        if rem != 0:
            cur = 0
            while True:
                t = argmax_first(x[b, cur])
                out.append(t)
                child = int(first_child[b, cur])
                while child != -1 and int(draft[b, child]) != t:
                    child = int(next_sibling[b, child])
                if child != -1:
                    acc += 1                          # t is an accepted draft
                if (eos is not None and t == eos) or (rem is not None and len(out) == rem) or child == -1:
                    break
                nodes.append(child)
                cur = child
        e = len(out)
        accept_len[b] = acc
        emit_count[b] = e
        out_tokens[b, :e] = out
        kept = nodes[:e]                          # nodes whose rows were read: one KV slot per emitted token
        path[b, :len(kept)] = kept
        status[b] = st
    offsets = np.zeros(B + 1, np.int32)
    offsets[1:] = np.cumsum(emit_count)
    return dict(accept_len=accept_len, emit_count=emit_count, out_tokens=out_tokens, path=path,
                emit_offsets=offsets, status=status)


def compact_tree_slots(kv, E: int, path, emit_count) -> np.ndarray:
    """Copy of kv [L, 2, B, H, C, D] where each sequence's kept tree slots
    (columns E + path[b, j]) are moved, in path order, to columns E + j for
    j < emit_count[b].  Other cells keep their bytes."""
    new = kv.copy()
    B = kv.shape[2]
    for b in range(B):
        for j in range(int(emit_count[b])):
            new[:, :, b, :, E + j, :] = kv[:, :, b, :, E + int(path[b, j]), :]
    return new


def chain_links(B: int, N: int):
    """first_child / next_sibling of a linear chain 0 -> 1 -> ... -> N-1."""
    fc = np.full((B, N), -1, np.int32)
    fc[:, :N - 1] = np.arange(1, N)
    return fc, np.full((B, N), -1, np.int32)
