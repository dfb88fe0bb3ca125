"""Greedy verification (oracle).  TEST INFRASTRUCTURE ONLY.

Row alignment ([Walkthrough] 3.3, alignment table): with a confirmed prefix of
length L and k proposals, one target forward over prefix + proposals gives a
row per input position; row i predicts the token at i + 1, so rows
L-1 .. L+k-2 verify proposals 1..k and row L+k-1 supplies the bonus.  The
verify step therefore sees exactly k + 1 rows per sequence, row j verifying
draft j (0-based) and row k being the bonus row.

Commit rule ([Walkthrough] 4.1 greedy commitment; [Forensics] App. D
BatchVerify; [Design] Standard Greedy Algorithm steps 3-6): walk the drafts in
order, emitting the target's argmax at each row; stop after emitting EOS or
after the output budget is used up; stop after the first row whose argmax
differs from the draft (that argmax is the correction); if every draft
matched, emit the bonus row's argmax as well.  A zero budget emits nothing.

Tie rule (reading of [Forensics] 4.2, which names argmax tie-breaking as a
divergence source without fixing it): the lowest index among equal maxima
wins; +0 and -0 are equal; an all -inf row gives index 0; NaN is unsupported.
"""
from __future__ import annotations

import numpy as np

from .status import ST_DRAFT_OOR


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def argmax_first(row: np.ndarray) -> int:
    """Index of the first maximal element of a float row.

    numpy's argmax returns the first occurrence of the maximum and compares
    with IEEE ordering, in which -0 == +0, which is the tie rule stated above.
    """
    return int(np.argmax(row))


def greedy_commit(rows: np.ndarray, proposals, remaining=None, eos_id=None):
    """One sequence, one round.  rows: [k+1, V] floats; proposals: k ids.

    Returns (emitted tokens, number of accepted drafts).
    """
    k = len(proposals)
    if remaining is not None and remaining == 0:
        return [], 0
    out = []
    accepted = 0
    for j in range(k):
        t = argmax_first(rows[j])
        out.append(t)
        if t == int(proposals[j]):
            accepted += 1
        if (eos_id is not None and t == eos_id) or (remaining is not None and len(out) == remaining):
            return out, accepted
        if t != int(proposals[j]):
            return out, accepted
    out.append(argmax_first(rows[k]))
    return out, accepted


def verification_rows(all_rows: np.ndarray, prefix_len: int) -> np.ndarray:
    """Rows of a full-prefix target forward that verify a round: rows[L-1:]."""
    return all_rows[prefix_len - 1:]


def greedy_verify(logits: np.ndarray, dtype: str, drafts: np.ndarray,
                  eos_id: int = -1, remaining=None) -> dict:
    """Batched greedy verify.

    logits: [B, k+1, V] float32, or uint16 bf16 bits when dtype == "bf16".
    drafts: [B, k] ints.  eos_id < 0 means no EOS.  remaining: None or [B].
    Returns accept_len, emit_count, out_tokens [B, k+1] (-1 padded),
    emit_offsets [B+1] (exclusive prefix sum of emit_count), status [B].
    """
    B, kp1, V = logits.shape
    k = kp1 - 1
    rows = widen_bf16(logits) if dtype == "bf16" else np.asarray(logits, dtype=np.float32)
    eos = None if eos_id < 0 else int(eos_id)
    accept_len = np.zeros(B, np.int32)
    emit_count = np.zeros(B, np.int32)
    out_tokens = np.full((B, kp1), -1, np.int32)
    status = np.zeros(B, np.int32)
    for b in range(B):
        d = [int(x) for x in drafts[b]]
        if any(x < 0 or x >= V for x in d):
            status[b] |= ST_DRAFT_OOR
        rem = None if remaining is None else int(remaining[b])
        toks, acc = greedy_commit(rows[b], d, rem, eos)
        accept_len[b] = acc
        emit_count[b] = len(toks)
        out_tokens[b, :len(toks)] = toks
    emit_offsets = np.zeros(B + 1, np.int32)
    for b in range(B):
        emit_offsets[b + 1] = emit_offsets[b] + emit_count[b]
    return dict(accept_len=accept_len, emit_count=emit_count, out_tokens=out_tokens,
                emit_offsets=emit_offsets, status=status)
