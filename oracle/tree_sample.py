"""Stochastic verification of a candidate tree (oracle).  TEST INFRASTRUCTURE
ONLY.

The pages name tree-structured verification ([Forensics] section 5) and list
what a tree verifier records, the draft tokens and their draft probabilities
among them ([Walkthrough] 5.2), but give no rule for verifying a tree by
sampling.  Reading used here: the published multi-draft form of speculative
sampling, in which the children of a node, drawn independently from the
draft's distribution q at that node, are tried one after another against a
target distribution that shrinks to the normalised positive residual after
every rejection.  Each try is one step of the rule of [Atlas] "Acceptance and
rejection correction" / [Walkthrough] 5.1 applied to the current residual, so
by induction the emitted token at every node is distributed as the target's
row there.

  * Trees as in oracle/tree.py: N nodes in topological order, node 0 the root,
    node i > 0 proposing draft[b, i]; first_child / next_sibling list each
    node's children in order (links must point forward inside the tree).
  * p[b, i] is the target's distribution after the path ending at node i;
    q[b, i] the draft's distribution at node i, from which node i's children
    were drawn (unused at a leaf).  Both float32, used as given.
  * Uniforms [B, N]: u[b, c] (c >= 1) decides the try of child c; u[b, 0] is
    the single draw (the correction, or the bonus at a leaf).
  * At the current node, with i rejections so far, the residual mass vector is
        R_0 = p_cur (float32),
        R_1 = max(p_cur - q_cur, 0) elementwise in float32,
        R_j = max(R_{j-1} - q_cur * m_{j-1}, 0) in float64 (j >= 2),
    with m_j = sum(R_j) correctly rounded (float64); the normalised residual
    is R_i / m_i (R_0 is used as it is).  The try of child x accepts when
    u < a: for i = 0, a = min(1, p(x) / q(x)) as one float32 division (the
    linear rule); for i >= 1, a = min(1, R_i(x) / (m_i * q(x))) in float64.
    q(x) == 0 gives a = 1 if the numerator is positive, else 0 (status);
    a draft id outside [0, V) is rejected (status).
  * A rejection moves to R_{i+1}.  If its mass is zero the residual stays
    R_i (status SPEC_ST_RESID_ZERO); if it is not finite the round emits
    token 0 and stops (status SPEC_ST_NONFINITE).
  * An accepted child's token is emitted and the child becomes the current
    node (its residual starts again at R_0 = its p row); EOS and the budget
    stop the round as in greedy verification.  When no child is accepted
    (or the node is a leaf) one token is drawn from the current R with u[b, 0]
    (the inverse CDF of oracle/sample.py: smallest v whose float64 prefix
    exceeds u * S, S its correctly rounded sum) and the round stops; a row
    with no positive mass gives token 0.
  * The kept KV slots are those of the nodes whose rows were read (the root
    and the accepted nodes), one per emitted token, as for greedy trees.

A chain tree (node i's only child is node i + 1) is exactly the linear
stochastic verification of oracle/sample.py.
"""
from __future__ import annotations

import math

import numpy as np

from .sample import accept_probability, draw_from_mass
from .status import ST_BAD_STATE, ST_DRAFT_OOR, ST_NONFINITE, ST_Q_ZERO, ST_RESID_ZERO


def _links_ok(first_child, next_sibling, N: int) -> bool:
    for i in range(N):
        for link in (int(first_child[i]), int(next_sibling[i])):
            if link != -1 and not (i < link < N):
                return False
    return True


def _draw64(R: np.ndarray, S: float, u) -> int | None:
    """Inverse-CDF draw from the float64 mass vector R of sum S."""
    if not (S > 0.0) or not math.isfinite(S):
        return None
    R = np.asarray(R, np.float64)
    T = float(np.float64(np.float32(u))) * S
    prefix = np.cumsum(R)
    v = int(np.searchsorted(prefix, T, side="right"))
    if v >= R.size:
        v = int(np.nonzero(R > 0.0)[0][-1])
    return v


def next_residual(R, m: float, i: int, p_row: np.ndarray, q_row: np.ndarray):
    """(R_{i+1}, m_{i+1}) after a rejection at residual R_i of mass m_i."""
    if i == 0:
        Rn = np.maximum(p_row - q_row, np.float32(0.0))        # float32, as the linear rule
        return Rn, math.fsum(Rn.astype(np.float64))
    Rn = np.maximum(np.asarray(R, np.float64) - q_row.astype(np.float64) * m, 0.0)
    return Rn, math.fsum(Rn)


def tree_sample_verify(p: np.ndarray, q: np.ndarray, draft, first_child, next_sibling, uniforms,
                       eos_id: int = -1, remaining=None) -> dict:
    """p, q [B, N, V] float32; draft, first_child, next_sibling [B, N] int;
    uniforms [B, N] float32.  Returns accept_len, emit_count, out_tokens
    [B, N] (-1 padded), path [B, N] (-1 padded), emit_offsets [B+1],
    final_mass [B] (S of the vector drawn from, 0 without a draw), status [B]."""
    p = np.asarray(p, np.float32)
    q = np.asarray(q, np.float32)
    B, N, V = p.shape
    eos = None if eos_id < 0 else int(eos_id)
    accept_len = np.zeros(B, np.int32)
    emit_count = np.zeros(B, np.int32)
    out_tokens = np.full((B, N), -1, np.int32)
    path = np.full((B, N), -1, np.int32)
    final_mass = np.zeros(B, np.float64)
    status = np.zeros(B, np.int32)
    for b in range(B):
        if not _links_ok(first_child[b], next_sibling[b], N):
            status[b] = ST_BAD_STATE
            continue
        rem = None if remaining is None else int(remaining[b])
        if rem == 0:
            continue
        u0 = uniforms[b, 0]
        out, nodes, acc, st = [], [0], 0, 0
        cur = 0
        while True:
            R, m, i = p[b, cur], 1.0, 0          # R_i and its mass m_i (R_0 used as given)
            accepted, stop = -1, False
            child = int(first_child[b, cur])
            while child != -1:
                x = int(draft[b, child])
                if not 0 <= x < V:
                    a_ok = False
                    st |= ST_DRAFT_OOR
                elif i == 0:
                    a, s = accept_probability(p[b, cur, x], q[b, cur, x])
                    st |= s
                    a_ok = bool(np.float32(uniforms[b, child]) < a)
                else:
                    qx = float(q[b, cur, x])
                    rx = float(R[x])
                    if not (math.isfinite(qx) and math.isfinite(rx)):
                        st |= ST_NONFINITE
                    if qx == 0.0:
                        a = 1.0 if rx > 0.0 else 0.0
                        st |= ST_Q_ZERO
                    else:
                        a = min(1.0, rx / (m * qx))
                    a_ok = float(np.float64(np.float32(uniforms[b, child]))) < a
                if a_ok:
                    accepted = child
                    break
                Rn, mn = next_residual(R, m, i, p[b, cur], q[b, cur])   # rejected
                if not math.isfinite(mn):
                    st |= ST_NONFINITE
                    stop, stop_mass = True, mn
                    break
                if mn > 0.0:
                    R, m, i = Rn, mn, i + 1
                else:
                    st |= ST_RESID_ZERO
                child = int(next_sibling[b, child])
            if stop:                               # a residual's mass is not finite
                out.append(0)
                final_mass[b] = stop_mass
                break
            if accepted != -1:
                x = int(draft[b, accepted])
                out.append(x)
                acc += 1
                if (eos is not None and x == eos) or (rem is not None and len(out) == rem):
                    break
                nodes.append(accepted)
                cur = accepted
                continue
            # no child accepted (or a leaf): one draw from the current residual
            if i == 0:
                tok, S = draw_from_mass(R, u0)
            else:
                S = m
                tok = _draw64(R, S, u0)
            if tok is None:
                if not math.isfinite(S):
                    st |= ST_NONFINITE
                else:
                    st |= ST_RESID_ZERO
                tok = 0
            out.append(int(tok))
            final_mass[b] = S
            break
        e = len(out)
        accept_len[b] = acc
        emit_count[b] = e
        out_tokens[b, :e] = out
        kept = nodes[:e]
        path[b, :len(kept)] = kept
        status[b] = st
    offsets = np.zeros(B + 1, np.int32)
    offsets[1:] = np.cumsum(emit_count)
    return dict(accept_len=accept_len, emit_count=emit_count, out_tokens=out_tokens, path=path,
                emit_offsets=offsets, final_mass=final_mass, status=status)
