"""Stochastic (Leviathan-style) verification (oracle).  TEST INFRASTRUCTURE ONLY.

Algorithm, in the order of [Atlas] "The mechanism" steps 2-5 and
[Walkthrough] 5.1:
  for each draft position j = 0..k-1 with proposed token x = d[b, j]:
    a = min(1, p_j(x) / q_j(x))                       ([Atlas] Acceptance and
                                                       rejection correction, a(x))
    accept x when the uniform u[b, j] is below a;     ([Walkthrough] 5.1 compares a
                                                       uniform draw with a, strictly)
    at the first rejection draw the correction from the positive residual
    r = max(p_j - q_j, 0), normalised by its mass,    ([Atlas] r(x))
    and discard the later drafts;
  after accepting every draft, draw one bonus token from the target row p_k.
EOS and the output budget stop the round as in greedy verification
([Walkthrough] 4.1).

Precision and randomness (readings, see the design notes):
  * p, q are float32 rows used as given (no renormalisation).  The acceptance
    ratio is one IEEE float32 division, capped at 1.  q(x) == 0 gives a = 1 if
    p(x) > 0 else 0 (status bit); a draft id outside [0, V) is rejected.
  * The random numbers are inputs: u[b, j] (j < k) decides acceptance at j and
    u[b, k] is the single draw used for the correction or the bonus.
  * A draw from a non-negative float32 mass vector r with uniform u takes
    S = sum(r) correctly rounded (math.fsum), T = u * S in float64, and returns
    the smallest v whose float64 inclusive prefix sum exceeds T (so tokens
    with zero mass are never chosen).  If rounding leaves no such v, the last v
    with positive mass is returned.
  * If the residual has no positive mass the draw falls back to p_j itself
    (status bit); a row with no positive mass at all yields token 0.
"""
from __future__ import annotations

import math

import numpy as np

from .status import ST_DRAFT_OOR, ST_NONFINITE, ST_Q_ZERO, ST_RESID_ZERO


def accept_probability(p_x, q_x):
    """(a, status) with a = min(1, p(x)/q(x)) in float32."""
    p32 = np.float32(p_x)
    q32 = np.float32(q_x)
    st = 0
    if not (np.isfinite(p32) and np.isfinite(q32)):
        st |= ST_NONFINITE
    if q32 == 0:
        return np.float32(1.0 if p32 > 0 else 0.0), st | ST_Q_ZERO
    ratio = np.float32(p32 / q32)
    return (ratio if ratio < np.float32(1.0) else np.float32(1.0)), st


def draw_from_mass(r: np.ndarray, u) -> tuple:
    """(token, S) for one draw from the unnormalised float32 mass vector r.

    token is None when S is not positive and finite.
    """
    r64 = np.asarray(r, dtype=np.float32).astype(np.float64)
    S = math.fsum(r64)
    if not (S > 0.0) or not math.isfinite(S):
        return None, S
    T = float(np.float64(np.float32(u))) * S
    prefix = np.cumsum(r64)
    v = int(np.searchsorted(prefix, T, side="right"))
    if v >= r64.size:
        v = int(np.nonzero(r64 > 0.0)[0][-1])
    return v, S


def _residual(p_row: np.ndarray, q_row: np.ndarray) -> np.ndarray:
    """Positive residual max(p - q, 0), elementwise in float32."""
    return np.maximum(p_row - q_row, np.float32(0.0))


def _bonus_row(p: np.ndarray, b: int, k: int) -> np.ndarray:
    """The row the bonus token is drawn from: the target's last row."""
    return p[b, k]


def _draw_row(row, u, fallback_row=None):
    """Draw from row (and from fallback_row if row has no positive mass)."""
    st = 0
    tok, S = draw_from_mass(row, u)
    if tok is None and not math.isfinite(S):
        return 0, S, ST_NONFINITE
    if tok is None:
        st |= ST_RESID_ZERO
        if fallback_row is not None:
            tok, S = draw_from_mass(fallback_row, u)
            if tok is None and not math.isfinite(S):
                return 0, S, st | ST_NONFINITE
        if tok is None:
            tok = 0
    return tok, S, st


def sample_verify(p: np.ndarray, q: np.ndarray, drafts: np.ndarray, uniforms: np.ndarray,
                  eos_id: int = -1, remaining=None) -> dict:
    """Batched stochastic verify.

    p: [B, k+1, V] float32, q: [B, k, V] float32, drafts: [B, k], uniforms:
    [B, k+1] float32 in [0, 1).  Returns accept_len, emit_count, out_tokens
    [B, k+1] (-1 padded), emit_offsets [B+1], final_mass [B] (float64 S of the
    row drawn from, 0 when no draw happened) and status [B].
    """
    B, kp1, V = p.shape
    k = kp1 - 1
    eos = None if eos_id < 0 else int(eos_id)
    accept_len = np.zeros(B, np.int32)
    emit_count = np.zeros(B, np.int32)
    out_tokens = np.full((B, kp1), -1, np.int32)
    final_mass = np.zeros(B, np.float64)
    status = np.zeros(B, np.int32)
    for b in range(B):
        rem = None if remaining is None else int(remaining[b])
        if rem is not None and rem == 0:
            continue
        out = []
        acc = 0
        st = 0
        stopped = False
        u_final = uniforms[b, k]
        for j in range(k):
            x = int(drafts[b, j])
            if 0 <= x < V:
                a, s = accept_probability(p[b, j, x], q[b, j, x])
                st |= s
            else:
                a = np.float32(0.0)
                st |= ST_DRAFT_OOR
            if np.float32(uniforms[b, j]) < a:
                out.append(x)
                acc += 1
                if (eos is not None and x == eos) or (rem is not None and len(out) == rem):
                    stopped = True
                    break
            else:
                resid = _residual(p[b, j], q[b, j])
                tok, S, s = _draw_row(resid, u_final, fallback_row=p[b, j])
                st |= s
                out.append(tok)
                final_mass[b] = S
                stopped = True
                break
        if not stopped:
            tok, S, s = _draw_row(_bonus_row(p, b, k), u_final)
            st |= s
            out.append(tok)
            final_mass[b] = S
        accept_len[b] = acc
        emit_count[b] = len(out)
        out_tokens[b, :len(out)] = out
        status[b] = st
    emit_offsets = np.zeros(B + 1, np.int32)
    for b in range(B):
        emit_offsets[b + 1] = emit_offsets[b] + emit_count[b]
    return dict(accept_len=accept_len, emit_count=emit_count, out_tokens=out_tokens,
                emit_offsets=emit_offsets, final_mass=final_mass, status=status)
