"""Pins for the paged (variable-length) commit oracle.

The paged layout must hold exactly what the contiguous layout holds after the
same rounds (both against per-sequence decoding: [Forensics] I2 applies to
either layout, App. F); page accounting must be exact; a commit that skips
the rollback must be caught.
"""
import numpy as np
import pytest

import oracle
from oracle.paged import commit_paged, gather_rows, pages_for, write_rows
from workloads import fill_kv_np, kv_bits_np, planted_greedy, write_forward_slots_np


def _content(b, pos, tok):
    d = np.arange(8)
    return kv_bits_np(b, np.asarray(pos)[:, None], np.asarray(tok)[:, None], 0, d[None, :], "bf16")


class _Paged:
    """A paged cache of one plane: pool [num_pages, page, 8] plus a free list."""

    def __init__(self, model, page, max_pages, num_pages, rng):
        self.page, self.max_pages = page, max_pages
        self.pool = np.zeros((num_pages, page, 8), np.uint16)
        self.free = list(rng.permutation(num_pages))
        self.bt = np.full((model.B, max_pages), -1, np.int32)
        self.owned = [0] * model.B
        for b in range(model.B):
            n = model.n(b)
            self.ensure(b, n)
            write_rows(self.pool, self.bt, b, np.arange(n), _content(b, np.arange(n), model.tokens[b][:n]), page)

    def ensure(self, b, rows):
        while self.owned[b] < pages_for(rows, self.page):
            self.bt[b, self.owned[b]] = self.free.pop(0)
            self.owned[b] += 1

    def release(self, out):
        for b in range(len(self.owned)):
            lo, hi = out["freed_offsets"][b], out["freed_offsets"][b + 1]
            got = list(out["freed"][lo:hi])
            assert got == list(self.bt[b, out["pages_kept"][b]:self.owned[b]])
            self.bt[b, out["pages_kept"][b]:self.owned[b]] = -1
            self.owned[b] = int(out["pages_kept"][b])
            self.free.extend(got)


@pytest.mark.parametrize("page", [1, 3, 16, 64])
def test_paged_and_contiguous_hold_the_same_rows(page):
    rng = np.random.default_rng(page)
    B, k, V, R = 5, 4, 50, 12
    P = rng.integers(2, 20, B)
    toks = [rng.integers(0, V, int(p)).tolist() for p in P]
    model = oracle.UnbatchedModel(toks)
    n = model.n_all()
    E = int(n.max())
    C = E + (k + 1) * R
    grid = np.zeros((B, int(P.max())), np.int64)
    for b in range(B):
        grid[b, :len(toks[b])] = toks[b]
    kv = fill_kv_np(1, 1, 8, B, C, E, n, grid, "bf16")              # plane 0 = (layer 0, K, head 0)
    max_pages = pages_for(int(P.max()) + (k + 1) * R + k + 1, page)
    pg = _Paged(model, page, max_pages, B * max_pages + 4, rng)
    for r in range(R):
        g = planted_greedy(rng, rng, B, k, V, 1.0, "f32", rng.uniform(0.2, 1.0, B))
        slots = model.slot_tokens(g["drafts"])
        n = model.n_all()
        write_forward_slots_np(kv, E, n, slots, "bf16")
        for b in range(B):                                          # the forward writes k+1 rows per sequence
            pg.ensure(b, n[b] + k + 1)
            pos = n[b] + np.arange(k + 1)
            write_rows(pg.pool, pg.bt, b, pos, _content(b, pos, slots[b]), page)
        ver = oracle.greedy_verify(g["logits"], "f32", g["drafts"])
        com = oracle.commit_realign(kv, E, n, ver["emit_count"], k)
        out = commit_paged(n, ver["emit_count"], k, page, pg.bt)
        assert (out["status"] == 0).all() and out["bytes_moved"] == 0
        assert np.array_equal(out["kv_len"], com["n_new"])
        pg.release(out)
        model.commit(ver["out_tokens"], ver["emit_count"])
        kv, E = com["kv"], com["E_new"]
        for b in range(B):
            nb = model.n(b)
            rows = gather_rows(pg.pool, pg.bt, b, nb, page)
            assert np.array_equal(rows, kv[0, 0, b, 0, E - nb:E, :]), (r, b)          # same as contiguous
            assert np.array_equal(rows, _content(b, np.arange(nb), model.tokens[b][:nb]))  # I2
        owned = [int(x) for b in range(B) for x in pg.bt[b, :pg.owned[b]]]
        assert len(set(owned)) == len(owned) and not set(owned) & set(pg.free)
        assert len(owned) + len(pg.free) == pg.pool.shape[0]


def test_page_counts_and_special_cases():
    bt = np.arange(4 * 6, dtype=np.int32).reshape(4, 6)
    out = commit_paged([0, 5, 7, 9], [0, 1, 5, 3], 4, 4, bt)
    # used pages ceil((n+5)/4) = 2, 3, 3, 4; kept ceil((n+e)/4) = 0, 2, 3, 3
    assert out["kv_len"].tolist() == [0, 6, 12, 12]
    assert out["pages_kept"].tolist() == [0, 2, 3, 3]
    assert out["freed"].tolist() == [0, 1, 8, 21]
    assert out["freed_offsets"].tolist() == [0, 2, 3, 3, 4]
    one = commit_paged([3], [2], 4, 1, np.arange(10, dtype=np.int32)[None])
    assert one["freed"].tolist() == [5, 6, 7]                     # page size 1: each rejected slot
    big = commit_paged([3], [1], 4, 64, np.arange(2, dtype=np.int32)[None])
    assert big["freed"].tolist() == [] and big["pages_kept"].tolist() == [1]


def test_invalid_sequences_release_nothing():
    bt = np.arange(3 * 3, dtype=np.int32).reshape(3, 3)
    out = commit_paged([5, -1, 3], [2, 1, 7], 3, 4, bt)
    assert out["status"].tolist() == [0, oracle.ST_BAD_STATE, oracle.ST_BAD_STATE]
    assert out["kv_len"].tolist() == [7, -1, 3]
    out = commit_paged([5], [1], 3, 4, np.arange(2, dtype=np.int32)[None])   # needs 3 pages, has 2
    assert out["status"].tolist() == [oracle.ST_CAPACITY] and out["freed"].size == 0


def test_negative_control_no_rollback():
    """Keeping all k+1 forward rows (no rollback) leaves a rejected draft's KV
    at a committed position once the next round overwrites only e rows."""
    rng = np.random.default_rng(9)
    model = oracle.UnbatchedModel([[3, 4, 5]])
    page, k = 4, 3
    pg = _Paged(model, page, 4, 8, rng)
    g = planted_greedy(rng, rng, 1, k, 20, 1.0, "f32", np.array([0.0]))   # first draft rejected
    slots = model.slot_tokens(g["drafts"])
    pg.ensure(0, model.n(0) + k + 1)
    write_rows(pg.pool, pg.bt, 0, model.n(0) + np.arange(k + 1), _content(0, model.n(0) + np.arange(k + 1), slots[0]), page)
    ver = oracle.greedy_verify(g["logits"], "f32", g["drafts"])
    assert ver["emit_count"][0] == 1
    wrong_len = model.n(0) + k + 1
    model.commit(ver["out_tokens"], ver["emit_count"])
    rows = gather_rows(pg.pool, pg.bt, 0, min(wrong_len, model.n(0) + 1), page)
    want = _content(0, np.arange(len(rows)), (model.tokens[0] + [-1])[:len(rows)])
    assert not np.array_equal(rows, want)
