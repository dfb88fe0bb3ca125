"""Per-sequence ("batch size one") reference state.  TEST INFRASTRUCTURE ONLY.

[Forensics] section 1 / 4.2 judge batched speculative decoding against each
sequence decoded on its own.  Here each sequence is just its list of
confirmed tokens; its KV cache holds one entry per confirmed token except
the last (which is fed to the next forward).  The KV entry of a token is a
pure function content(b, position, token, plane, d) supplied by the caller,
standing in for the target model.

check() tests the three invariants of [Forensics] section 3 on a batched
state (kv, pos, mask, E):
  I1  rectangular alignment: sequence b's mask is 1 exactly on the n_b
      columns ending at E, 0 elsewhere;
  contiguity: position ids are 0..n_b-1 over those columns, 0 elsewhere;
  I2  every unmasked cell holds content(b, pos, token at pos) -- so a cell
      kept from a rejected draft, or left at an old column, is caught.
"""
from __future__ import annotations

import numpy as np


class UnbatchedModel:
    def __init__(self, tokens):
        self.tokens = [list(int(x) for x in t) for t in tokens]

    @property
    def B(self) -> int:
        return len(self.tokens)

    def n(self, b: int) -> int:
        return len(self.tokens[b]) - 1

    def n_all(self) -> np.ndarray:
        return np.array([self.n(b) for b in range(self.B)], np.int64)

    def slot_tokens(self, drafts) -> np.ndarray:
        """Tokens whose KV the verify forward writes into slots 0..k."""
        return np.array([[self.tokens[b][-1]] + [int(x) for x in drafts[b]]
                         for b in range(self.B)], np.int64)

    def commit(self, out_tokens, emit_count) -> None:
        for b in range(self.B):
            self.tokens[b].extend(int(x) for x in out_tokens[b][:int(emit_count[b])])

    def check(self, kv, pos, mask, E: int, content, lag=None) -> list:
        """List of violated invariants (empty when the state is correct).

        kv: element bits [L, 2, B, H, C, D]; content(b, pos, tok, plane, d)
        returns element bits broadcast over its arguments.  lag[b] (default 0)
        is how many more confirmed tokens this cache lacks beyond the last one
        (a draft cache after full acceptance lacks one).  pos / mask may be
        None to skip their checks.
        """
        L, _, B, H, C, D = kv.shape
        bad = []
        for b in range(B):
            n = self.n(b) - (0 if lag is None else int(lag[b]))
            want_mask = np.zeros(C, np.int32)
            want_mask[E - n:E] = 1
            if mask is not None and not np.array_equal(mask[b], want_mask):
                bad.append(f"I1 mask b={b}")
            want_pos = np.zeros(C, np.int32)
            want_pos[E - n:E] = np.arange(n, dtype=np.int32)
            if pos is not None and not np.array_equal(pos[b], want_pos):
                bad.append(f"contiguity pos b={b}")
            if n == 0:
                continue
            p = np.arange(n, dtype=np.int64)
            tok = np.array(self.tokens[b][:n], np.int64)
            plane = np.arange(L * 2 * H, dtype=np.int64).reshape(L, 2, H)
            want = content(b, p[None, None, None, :, None], tok[None, None, None, :, None],
                           plane[:, :, :, None, None], np.arange(D)[None, None, None, None, :])
            got = kv[:, :, b, :, E - n:E, :]
            if not np.array_equal(got, want):
                bad.append(f"I2 kv b={b}")
        return bad


def check_ragged(tokens, pool, n, content) -> list:
    """Invariants of a ragged pool [L, 2, N, H, Cs, D] ([Forensics] 3.2: EXSPEC
    keeps sequences ragged): sequence s holds exactly n_s = len(tokens[s]) - 1
    rows at columns [0, n_s), each the KV of (s, position, token at that
    position).  content(s, pos, tok, plane, d) as in UnbatchedModel.check."""
    L, _, N, H, Cs, D = pool.shape
    bad = []
    plane = np.arange(L * 2 * H, dtype=np.int64).reshape(L, 2, H)
    for s in range(N):
        ns = len(tokens[s]) - 1
        if int(n[s]) != ns:
            bad.append(f"length s={s}")
            continue
        if ns == 0:
            continue
        p = np.arange(ns, dtype=np.int64)
        tok = np.array(tokens[s][:ns], np.int64)
        want = content(s, p[None, None, None, :, None], tok[None, None, None, :, None],
                       plane[:, :, :, None, None], np.arange(D)[None, None, None, None, :])
        if not np.array_equal(pool[:, :, s, :, 0:ns, :], want):
            bad.append(f"I2 pool s={s}")
    return bad
