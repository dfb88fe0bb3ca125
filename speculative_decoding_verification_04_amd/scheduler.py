"""Multi-round EQSPEC and EXSPEC schedulers over the library's calls.

[Forensics] 3.1: EQSPEC keeps each batch rectangular and realigns it after
every verification.  [Forensics] 3.2: EXSPEC keeps sequences ragged, batches
identical-length sequences from a window larger than the batch (no
realignment), and falls back to unpad-append-repad for a batch that is not
same-length.  [Forensics] 4.3 / Table 5 compare them by verification calls
and alignment overhead.

Both schedulers verify every pool sequence once per round (greedy), so they
emit the same tokens and differ in batching and in the KV bytes they move:
  * EqspecPool: fixed batches of B consecutive sequences, each a left-padded
    rectangle; per batch: spec_verify_greedy, then spec_commit_realign_kv.
  * ExspecPool: one ragged pool [L][2][N][H][Cs][D] (sequence s at columns
    [0, n_s)); per round spec_group_same_length over the pool's cached row
    counts; a same-length batch: spec_verify_greedy, then spec_commit_paged
    with one page per sequence (a length update: nothing moves); a mixed
    batch: spec_repad_kv into a rectangle right-aligned at the batch's
    longest sequence, spec_verify_greedy, spec_unpad_kv back into the pool.
The verify forward (the target model writing the k+1 slots' KV and producing
the logits) is the caller's: `forward(kv, rows, seq, col0, pos0, tokens)`
writes the slots, and each round's logits and drafts are given per pool
sequence.  Torch only allocates, indexes and moves small host values.

Every library call of a round is bracketed by HIP events, so a round reports
GPU time per step (grouping, verification, commit) apart from the forward.
"""
from __future__ import annotations

import numpy as np

from . import (spec_commit_paged, spec_commit_realign_kv, spec_group_same_length, spec_repad_kv,
               spec_unpad_kv, spec_verify_greedy, spec_verify_greedy_workspace_bytes, workspace,
               SPEC_BF16, SPEC_F32)


class _Timer:
    """HIP events around library calls, summed per label after a sync."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def __call__(self, label, fn):
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.marks.append((label, a, b))

    def totals(self) -> dict:
        self.torch.cuda.synchronize()
        out = {}
        for label, a, b in self.marks:
            out[label] = out.get(label, 0.0) + a.elapsed_time(b) * 1e-3
        self.marks = []
        return out


def _slot_tokens(tokens, members, drafts_h) -> np.ndarray:
    return np.array([[tokens[s][-1]] + [int(x) for x in drafts_h[s]] for s in members], np.int64)


class EqspecPool:
    """Fixed batches of B consecutive pool sequences, each its own rectangle."""

    def __init__(self, torch, tokens, L, H, D, dtype, k, B, C, V, device, fill):
        """fill(kv, E, n, seq) writes a rectangle's initial contents."""
        self.t, self.k, self.B, self.C = torch, k, B, C
        self.tokens = [list(x) for x in tokens]
        N = len(tokens)
        assert N % B == 0
        self.nb = N // B
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.dt = SPEC_BF16 if dtype == "bf16" else SPEC_F32
        n = np.array([len(x) - 1 for x in tokens], np.int64)
        self.n_h = n.copy()
        self.E_h = [int(n[i * B:(i + 1) * B].max()) for i in range(self.nb)]
        self.rects = torch.empty((self.nb, L, 2, B, H, C, D), dtype=tdt, device=device)
        for i in range(self.nb):
            fill(self.rects[i], self.E_h[i], n[i * B:(i + 1) * B], np.arange(i * B, (i + 1) * B))
        i32 = dict(dtype=torch.int32, device=device)
        self.E = [torch.tensor(self.E_h, **i32), torch.empty(self.nb, **i32)]
        self.n = [torch.as_tensor(n.astype(np.int32)).to(device), torch.empty(N, **i32)]
        self.pos, self.mask = torch.empty(B, C, **i32), torch.empty(B, C, **i32)
        self.moved = torch.zeros(self.nb, dtype=torch.int64, device=device)
        self.acc, self.emit = torch.empty(N, **i32), torch.empty(N, **i32)
        self.out = torch.empty(N, k + 1, **i32)
        self.ws = workspace(spec_verify_greedy_workspace_bytes(B, k, V, self.dt), device)
        self.timer = _Timer(torch)
        self.cur = 0

    def round(self, logits, drafts, drafts_h, forward) -> dict:
        B, k, c = self.B, self.k, self.cur
        for i in range(self.nb):
            m = slice(i * B, (i + 1) * B)
            members = np.arange(i * B, (i + 1) * B)
            forward(self.rects[i], np.arange(B), members, np.full(B, self.E_h[i]), self.n_h[m],
                    _slot_tokens(self.tokens, members, drafts_h))
            self.timer("verify", lambda: spec_verify_greedy(logits[m], drafts[m], self.acc[m], self.emit[m],
                                                            self.out[m], self.ws))
            self.timer("commit", lambda: spec_commit_realign_kv(
                self.rects[i], k, self.E[c][i:i + 1], self.n[c][m], self.emit[m], self.E[1 - c][i:i + 1],
                self.n[1 - c][m], self.pos, self.mask, bytes_moved=self.moved[i:i + 1]))
        times = self.timer.totals()
        self.cur = 1 - c
        emit = self.emit.cpu().numpy()
        out = self.out.cpu().numpy()
        self.n_h = self.n[self.cur].cpu().numpy().astype(np.int64)
        self.E_h = [int(x) for x in self.E[self.cur].cpu().numpy()]
        for s in range(len(self.tokens)):
            self.tokens[s].extend(int(x) for x in out[s][:emit[s]])
        return dict(emit_count=emit, out_tokens=out, verify_calls=self.nb,
                    bytes_moved=int(self.moved.sum().item()), times=times)


class ExspecPool:
    """Ragged per-sequence caches regrouped by length every round."""

    def __init__(self, torch, tokens, L, H, D, dtype, k, B, min_group, Cs, V, device, fill):
        """fill(pool, n) writes the pool's initial (ragged) contents."""
        self.t, self.k, self.B, self.min_group, self.Cs = torch, k, B, min_group, Cs
        self.L, self.H, self.D = L, H, D
        self.tokens = [list(x) for x in tokens]
        N = len(tokens)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.dt = SPEC_BF16 if dtype == "bf16" else SPEC_F32
        self.elt = 2 if dtype == "bf16" else 4
        n = np.array([len(x) - 1 for x in tokens], np.int64)
        self.n_h = n.copy()
        self.pool = torch.empty((L, 2, N, H, Cs, D), dtype=tdt, device=device)
        fill(self.pool, n)
        # fallback rectangles [L, 2, nb, H, Cs, D] (nb <= B members) share one buffer
        self.rect_store = torch.empty(L * 2 * B * H * Cs * D, dtype=tdt, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.dev = device
        self.n = torch.as_tensor(n.astype(np.int32)).to(device)
        self.perm, self.bstart = torch.empty(N, **i32), torch.empty(N + 1, **i32)
        self.blen, self.nbat, self.ngrp = torch.empty(N, **i32), torch.empty(1, **i32), torch.empty(1, **i32)
        self.acc, self.emit = torch.empty(B, **i32), torch.empty(B, **i32)
        self.out = torch.empty(B, k + 1, **i32)
        self.len_out, self.kept = torch.empty(B, **i32), torch.empty(B, **i32)
        self.freed, self.freed_off = torch.empty(B * (k + 1), **i32), torch.empty(B + 1, **i32)
        self.E = torch.empty(1, **i32)
        self.ws = workspace(spec_verify_greedy_workspace_bytes(B, k, max(V, 1), self.dt), device)
        self.timer = _Timer(torch)

    def round(self, logits, drafts, drafts_h, forward) -> dict:
        t, k = self.t, self.k
        N = len(self.tokens)
        self.timer("group", lambda: spec_group_same_length(self.n, self.B, self.min_group, self.perm, self.bstart,
                                                           self.blen, self.nbat, self.ngrp))
        nbat = int(self.nbat.item())
        perm = self.perm.cpu().numpy()
        bstart = self.bstart.cpu().numpy()
        blen = self.blen.cpu().numpy()
        emit_all = np.zeros(N, np.int32)
        out_all = np.full((N, k + 1), -1, np.int32)
        col_bytes = self.L * 2 * self.H * self.D * self.elt
        moved = mixed = 0
        for b in range(nbat):
            idx = perm[bstart[b]:bstart[b + 1]].astype(np.int64)
            nb = len(idx)
            idx_d = t.as_tensor(idx).to(self.dev)
            idx32 = idx_d.to(t.int32)
            lg = logits.index_select(0, idx_d)
            dr = drafts.index_select(0, idx_d)
            n_idx = self.n_h[idx].copy()
            n_d = t.as_tensor(n_idx.astype(np.int32)).to(self.dev)
            slots = _slot_tokens(self.tokens, idx, drafts_h)
            acc, emit, out = self.acc[:nb], self.emit[:nb], self.out[:nb]
            if blen[b] >= 0:
                forward(self.pool, idx, idx, n_idx, n_idx, slots)
                self.timer("verify", lambda: spec_verify_greedy(lg, dr, acc, emit, out, self.ws))
                self.timer("commit", lambda: spec_commit_paged(
                    k, self.Cs, n_d, emit, idx32.view(nb, 1), self.len_out[:nb], self.kept[:nb],
                    self.freed[:nb * (k + 1)], self.freed_off[:nb + 1]))
            else:
                mixed += 1
                E = int(n_idx.max())
                self.E.fill_(E)
                rect = self.rect_store[:self.L * 2 * nb * self.H * self.Cs * self.D].view(
                    self.L, 2, nb, self.H, self.Cs, self.D)
                self.timer("commit", lambda: spec_repad_kv(self.pool, rect, idx32, n_d, self.E))
                forward(rect, np.arange(nb), idx, np.full(nb, E), n_idx, slots)
                self.timer("verify", lambda: spec_verify_greedy(lg, dr, acc, emit, out, self.ws))
                self.timer("commit", lambda: spec_unpad_kv(rect, self.pool, idx32, n_d, emit, self.E,
                                                           self.len_out[:nb]))
            self.n.index_copy_(0, idx_d, self.len_out[:nb])
            e_h = emit.cpu().numpy()
            if blen[b] < 0:
                moved += 2 * int(n_idx.sum()) * col_bytes + 2 * int((n_idx + e_h).sum()) * col_bytes
            emit_all[idx] = e_h
            out_all[idx] = out.cpu().numpy()
            self.n_h[idx] = n_idx + e_h
        times = self.timer.totals()
        for s in range(N):
            self.tokens[s].extend(int(x) for x in out_all[s][:emit_all[s]])
        return dict(emit_count=emit_all, out_tokens=out_all, verify_calls=nbat, bytes_moved=moved,
                    mixed_batches=mixed, num_grouped=int(self.ngrp.item()), times=times)
