"""Pins of the ragged-cache copies and the multi-round EQSPEC / EXSPEC loop
(oracle/ragged.py, oracle/policy.py) against per-sequence decoding
([Forensics] section 3: the invariants; 3.2: EXSPEC keeps sequences ragged).

The loop is checked by what the pages fix rather than by retyping it: after
every round every sequence's cached rows hold exactly the KV of its own
committed tokens at their positions (UnbatchedModel / check_ragged), both
policies emit the same tokens (they verify the same inputs), a same-length
batch moves no KV bytes, and planted mistakes (a mixed batch committed by a
length update, a lost unpad) are caught."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.unbatched import check_ragged

DT = "f32"


def content(seq_map=None):
    def f(b, pos, tok, plane, d):
        s = b if seq_map is None else seq_map[b]
        return W.kv_bits_np(s, pos, tok, plane, d, DT)
    return f


def forward(kv, rows, seq, col0, pos0, tokens):
    W.write_rows_np(kv, rows, seq, col0, pos0, tokens, DT)


def test_repad_hand_example():
    # pool of 3 sequences, 1 plane of width 1: values are (sequence, row) labels
    pool = np.zeros((1, 2, 3, 1, 5, 1), np.uint32)
    for s in range(3):
        pool[:, :, s, :, :, 0] = 10 * (s + 1) + np.arange(5)
    rect = np.full((1, 2, 2, 1, 6, 1), 7, np.uint32)
    got = oracle.repad_kv(pool, rect, index=[2, 0], kv_len=[3, 1], E=4)
    assert got[0, 0, 0, 0, :, 0].tolist() == [7, 30, 31, 32, 7, 7]    # rows [E - 3, E) of sequence 2
    assert got[0, 0, 1, 0, :, 0].tolist() == [7, 7, 7, 10, 7, 7]      # one row of sequence 0
    # the forward writes slots at [E, E + k + 1); unpad keeps e of them
    got[0, :, 0, 0, 4:6, 0] = [90, 91]
    got[0, :, 1, 0, 4:6, 0] = [80, 81]
    u = oracle.unpad_kv(got, pool, index=[2, 0], kv_len=[3, 1], emit_count=[2, 1], E=4)
    assert u["pool"][0, 0, 2, 0, :, 0].tolist() == [30, 31, 32, 90, 91]
    assert u["pool"][0, 0, 0, 0, :, 0].tolist() == [10, 80, 12, 13, 14]
    assert u["pool"][0, 0, 1, 0, :, 0].tolist() == pool[0, 0, 1, 0, :, 0].tolist()
    assert u["kv_len"].tolist() == [5, 2]


def test_repad_unpad_round_trip_is_identity_on_cached_rows():
    rng = np.random.default_rng(3)
    L, N, H, Cs, D, B = 2, 9, 3, 40, 4, 4
    pool = rng.integers(0, 2 ** 32, size=(L, 2, N, H, Cs, D), dtype=np.uint32)
    idx = rng.choice(N, B, replace=False)
    n = rng.integers(0, 30, size=B)
    E = int(n.max()) + 2
    rect = rng.integers(0, 2 ** 32, size=(L, 2, B, H, 45, D), dtype=np.uint32)
    r = oracle.repad_kv(pool, rect, idx, n, E)
    u = oracle.unpad_kv(r, pool, idx, n, np.zeros(B, np.int32), E)
    assert np.array_equal(u["pool"], pool)
    assert oracle.ragged_bytes(n, np.zeros(B), 8)["repad"] == 2 * int(n.sum()) * 8


def _states(pool_P, B, k, L=1, H=2, D=4, seed=0):
    N = len(pool_P)
    rng = np.random.default_rng(seed)
    tokens = [list(rng.integers(0, 50, size=int(p))) for p in pool_P]
    n = np.asarray(pool_P, np.int64) - 1
    R_max = 8
    rects, Es = [], []
    for i in range(N // B):
        m = np.arange(i * B, (i + 1) * B)
        E = int(n[m].max())
        C = E + (k + 1) * (R_max + 1)
        t = np.zeros((B, int(pool_P.max()) + 1), np.int64)
        for j, s in enumerate(m):
            t[j, :len(tokens[s])] = tokens[s]
        rects.append(W.fill_kv_np(L, H, D, B, C, E, n[m], t, DT, seq=m))
        Es.append(E)
    Cs = int(n.max()) + (k + 1) * (R_max + 1)
    t = np.zeros((N, int(pool_P.max()) + 1), np.int64)
    for s in range(N):
        t[s, :len(tokens[s])] = tokens[s]
    pool = W.fill_kv_np(L, H, D, N, Cs, n, n, t, DT)
    eq = dict(rects=rects, E=Es, n=n.copy(), tokens=[list(x) for x in tokens], B=B)
    ex = dict(pool=pool, rect=np.zeros((L, 2, B, H, Cs, D), np.uint32), n=n.copy(),
              tokens=[list(x) for x in tokens], B=B, min_group=2)
    return eq, ex


def _check_eq(eq, B):
    bad = []
    for i, rect in enumerate(eq["rects"]):
        m = np.arange(i * B, (i + 1) * B)
        model = oracle.UnbatchedModel([eq["tokens"][s] for s in m])
        bad += model.check(rect, None, None, eq["E"][i], content(m))
    return bad


@pytest.mark.parametrize("lengths", ["spread", "few"])
def test_loop_keeps_every_sequence_equal_to_per_sequence_decoding(lengths):
    rng = np.random.default_rng(11)
    N, B, k, V = 16, 4, 3, 50
    P = rng.integers(5, 40, size=N) if lengths == "spread" else rng.choice([9, 10, 20], size=N)
    alpha = rng.uniform(0.3, 0.95, size=N)
    eq, ex = _states(P, B, k)
    saw_uniform = saw_mixed = False
    for r in range(6):
        g = W.policy_round(r, N, k, V, DT, 1.0, alpha)
        a = oracle.eqspec_round(eq, g["logits"], g["drafts"], DT, k, forward)
        b = oracle.exspec_round(ex, g["logits"], g["drafts"], DT, k, forward)
        assert np.array_equal(a["emit_count"], b["emit_count"])
        assert np.array_equal(a["out_tokens"], b["out_tokens"])
        assert eq["tokens"] == ex["tokens"]
        assert not _check_eq(eq, B)
        assert not check_ragged(ex["tokens"], ex["pool"], ex["n"], content())
        assert a["verify_calls"] == N // B
        gr = b["grouping"]
        saw_uniform |= gr["num_grouped"] > 0
        saw_mixed |= b["mixed_batches"] > 0
        # bytes: only mixed batches move KV (cached rows twice, plus kept slots)
        assert (b["bytes_moved"] == 0) == (b["mixed_batches"] == 0)
    assert saw_uniform and saw_mixed


def test_same_length_pool_moves_nothing_in_its_first_round():
    N, B, k, V = 8, 4, 2, 40
    P = np.full(N, 12)
    eq, ex = _states(P, B, k)
    g = W.policy_round(0, N, k, V, DT, 1.0, np.full(N, 0.6))
    b = oracle.exspec_round(ex, g["logits"], g["drafts"], DT, k, forward)
    assert b["mixed_batches"] == 0 and b["bytes_moved"] == 0 and b["verify_calls"] == 2
    assert not check_ragged(ex["tokens"], ex["pool"], ex["n"], content())


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(5)
    N, B, k, V = 12, 4, 3, 50
    P = rng.integers(5, 30, size=N)
    g = W.policy_round(0, N, k, V, DT, 1.0, np.full(N, 0.8))
    # 1. a mixed batch committed by a length update only (its slots went to the rectangle)
    _, ex = _states(P, B, k)
    import oracle.policy as pol
    real = pol.unpad_kv

    def lengths_only(rect, pool, index, kv_len, emit_count, E):
        return {"pool": pool, "kv_len": np.asarray(kv_len) + np.asarray(emit_count)}
    monkeypatch.setattr(pol, "unpad_kv", lengths_only)
    oracle.exspec_round(ex, g["logits"], g["drafts"], DT, k, forward)
    assert check_ragged(ex["tokens"], ex["pool"], ex["n"], content())
    # 2. unpad that keeps every forward slot (rejected drafts' KV appended)
    _, ex = _states(P, B, k)

    def keeps_all(rect, pool, index, kv_len, emit_count, E):
        return real(rect, pool, index, kv_len, np.full(len(index), k + 1), E)
    monkeypatch.setattr(pol, "unpad_kv", keeps_all)
    oracle.exspec_round(ex, g["logits"], g["drafts"], DT, k, forward)
    assert check_ragged(ex["tokens"], ex["pool"], ex["n"], content())
