"""Pins for the commit/realign oracle: no-op special cases, multi-round
invariants against per-sequence decoding, byte count, saturation law,
negative controls, invalid states."""
import numpy as np
import pytest

import oracle
from workloads import fill_kv_np, kv_bits_np, planted_greedy, write_forward_slots_np


def _content(dtype):
    return lambda b, pos, tok, plane, d: kv_bits_np(b, pos, tok, plane, d, dtype)


def _state(B=5, L=2, H=2, D=8, k=3, V=20, rounds=50, dtype="bf16", seed=0, lo=3, hi=12):
    rng = np.random.default_rng(seed)
    P = rng.integers(lo, hi + 1, size=B)
    toks = [rng.integers(0, V, size=int(p)).tolist() for p in P]
    model = oracle.UnbatchedModel(toks)
    n = model.n_all()
    E = int(n.max())
    C = E + (k + 1) * rounds
    tok_grid = np.zeros((B, int(P.max())), np.int64)
    for b in range(B):
        tok_grid[b, :len(toks[b])] = toks[b]
    kv = fill_kv_np(L, H, D, B, C, E, n, tok_grid, dtype)
    pos, mask = oracle.position_and_mask(E, n, C)
    return dict(model=model, kv=kv, pos=pos, mask=mask, E=E, C=C, k=k, V=V, dtype=dtype, rng=rng)


def _round(st, alpha=0.6, remaining=None, eos_id=-1, commit_e=None):
    """One verify + commit round with the oracle; returns the verify result."""
    model, kv, k, V = st["model"], st["kv"], st["k"], st["V"]
    B = model.B
    rng = st["rng"]
    r = planted_greedy(rng, rng, B, k, V, 1.0, "f32", alpha)
    write_forward_slots_np(kv, st["E"], model.n_all(), model.slot_tokens(r["drafts"]), st["dtype"])
    ver = oracle.greedy_verify(r["logits"], "f32", r["drafts"], eos_id=eos_id, remaining=remaining)
    e = ver["emit_count"] if commit_e is None else commit_e(ver["emit_count"])
    com = oracle.commit_realign(kv, st["E"], model.n_all(), e, k)
    assert com["ok"]
    model.commit(ver["out_tokens"], ver["emit_count"])
    st.update(kv=com["kv"], pos=com["pos"], mask=com["mask"], E=com["E_new"])
    return ver, com


def test_initial_state_satisfies_invariants():
    st = _state()
    assert st["model"].check(st["kv"], st["pos"], st["mask"], st["E"], _content("bf16")) == []


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fifty_rounds_invariants(dtype):
    st = _state(dtype=dtype, rounds=50)
    rng = np.random.default_rng(7)
    for r in range(50):
        rem = None
        if r % 5 == 4:   # exercise output budgets, including zero
            rem = rng.integers(0, st["k"] + 2, size=st["model"].B)
        _round(st, alpha=0.4 + 0.5 * (r % 3) / 2, remaining=rem, eos_id=(3 if r % 7 == 6 else -1))
        bad = st["model"].check(st["kv"], st["pos"], st["mask"], st["E"], _content(dtype))
        assert bad == [], (r, bad)


def test_noop_single_sequence_and_uniform_acceptance():
    """One sequence, or equal acceptance everywhere: padding unchanged, nothing moves."""
    for B, e in [(1, [3]), (4, [2, 2, 2, 2]), (3, [5, 5, 5])]:
        st = _state(B=B, k=4, rounds=2)
        kv0 = st["kv"].copy()
        n = st["model"].n_all()
        com = oracle.commit_realign(kv0, st["E"], n, e, 4)
        assert com["bytes_moved"] == 0
        assert (com["delta"] == 0).all()
        assert np.array_equal(com["kv"], kv0)
        # every sequence's range start column is unchanged
        assert np.array_equal(com["E_new"] - com["n_new"], st["E"] - n)


def test_bytes_moved_counts_cells_that_change_column():
    st = _state(B=6, rounds=3)
    n = st["model"].n_all()
    e = np.array([1, 4, 2, 4, 3, 0])
    com = oracle.commit_realign(st["kv"], st["E"], n, e, st["k"])
    L, _, B, H, C, D = st["kv"].shape
    col = L * 2 * H * D * st["kv"].itemsize
    moved_cells = 0
    for b in range(B):
        old_cols = np.arange(st["E"] - n[b], st["E"] + e[b])
        new_cols = np.nonzero(com["mask"][b])[0]
        assert len(old_cols) == len(new_cols)
        moved_cells += int((old_cols != new_cols).sum())
    assert com["bytes_moved"] == 2 * moved_cells * col


def test_padding_per_sequence_saturates():
    """Mean inserted padding per sequence, mean (M - e_b), rises with B and
    saturates at (k+1) - E[e] (forensics summary, App. B)."""
    k, a = 4, 0.7
    Ee = (1 - a ** (k + 1)) / (1 - a)
    rng = np.random.default_rng(3)
    means = []
    for B in [1, 2, 4, 8, 4096]:
        trials = []
        for _ in range(max(1, 40000 // B)):
            s = rng.random((B, k)) < a
            e = np.argmin(np.concatenate([s, np.zeros((B, 1), bool)], 1), 1) + 1
            bk = oracle.commit_bookkeeping(10, np.zeros(B, int), e, k, 10 + k + 1)
            trials.append(bk["delta"].mean())
        means.append(float(np.mean(trials)))
    assert means[0] == 0.0
    assert all(x < y for x, y in zip(means, means[1:]))       # rises with B ...
    assert abs(means[-1] - ((k + 1) - Ee)) < 0.02              # ... to (k+1) - E[e]


def test_negative_control_masking_only():
    """Updating mask and positions without moving the KV leaves it desynchronised."""
    st = _state(B=5)
    model = st["model"]
    # planting rates 0 and 1 force ragged acceptance (e = 1 and e = k + 1)
    r = planted_greedy(st["rng"], st["rng"], model.B, st["k"], st["V"], 1.0, "f32",
                       [0.0, 1.0, 0.6, 0.6, 0.6])
    write_forward_slots_np(st["kv"], st["E"], model.n_all(), model.slot_tokens(r["drafts"]), "bf16")
    ver = oracle.greedy_verify(r["logits"], "f32", r["drafts"])
    e = ver["emit_count"]
    assert e[0] == 1 and e[1] == st["k"] + 1
    com = oracle.commit_realign(st["kv"], st["E"], model.n_all(), e, st["k"])
    model.commit(ver["out_tokens"], e)
    bad = model.check(st["kv"], com["pos"], com["mask"], com["E_new"], _content("bf16"))
    assert any(x.startswith("I2") for x in bad)
    # the correct commit passes
    assert model.check(com["kv"], com["pos"], com["mask"], com["E_new"], _content("bf16")) == []


def test_negative_control_keep_rejected_kv():
    """Keeping one more slot than emitted keeps a rejected draft's KV."""
    st = _state(B=5)
    k = st["k"]
    ver, com = _round(st, alpha=0.3, commit_e=lambda e: np.minimum(e + 1, k + 1))
    bad = st["model"].check(st["kv"], st["pos"], st["mask"], st["E"], _content("bf16"))
    assert bad, "keeping rejected KV must violate the invariants"


def test_negative_control_stale_position_ids():
    st = _state(B=5)
    old_pos = st["pos"].copy()
    model = st["model"]
    r = planted_greedy(st["rng"], st["rng"], model.B, st["k"], st["V"], 1.0, "f32",
                       [1.0, 0.0, 0.5, 0.5, 0.5])
    write_forward_slots_np(st["kv"], st["E"], model.n_all(), model.slot_tokens(r["drafts"]), "bf16")
    ver = oracle.greedy_verify(r["logits"], "f32", r["drafts"])
    e = ver["emit_count"]
    com = oracle.commit_realign(st["kv"], st["E"], model.n_all(), e, st["k"])
    model.commit(ver["out_tokens"], e)
    stale = np.zeros_like(com["pos"])
    stale[:, :old_pos.shape[1]] = old_pos
    bad = model.check(com["kv"], stale, com["mask"], com["E_new"], _content("bf16"))
    assert any(x.startswith("contiguity") for x in bad)


@pytest.mark.parametrize("E,n,e,C,bits", [
    (10, [3, 4], [1, 2], 13, [oracle.ST_CAPACITY] * 2),      # E + k + 1 > C (k = 3)
    (-1, [0, 0], [1, 1], 20, [oracle.ST_CAPACITY | oracle.ST_BAD_STATE] * 2),
    (10, [11, 4], [1, 2], 30, [oracle.ST_BAD_STATE, 0]),
    (10, [3, 4], [5, 2], 30, [oracle.ST_BAD_STATE, 0]),
    (10, [3, -1], [1, -1], 30, [0, oracle.ST_BAD_STATE]),
])
def test_invalid_state_reports_status_only(E, n, e, C, bits):
    res = oracle.commit_realign(None, E, n, e, 3, C)
    assert not res["ok"]
    assert res["status"].tolist() == bits
    assert "pos" not in res and "kv" not in res


def _draft_round(st, alpha):
    """One round on a draft cache: the draft forward writes k slots (the last
    confirmed token and d_1..d_{k-1}); verification of the target decides e."""
    model, kv, k, V = st["model"], st["kv"], st["k"], st["V"]
    rng = st["rng"]
    r = planted_greedy(rng, rng, model.B, k, V, 1.0, "f32", alpha)
    slots = model.slot_tokens(r["drafts"])[:, :k]
    write_forward_slots_np(kv, st["E"], model.n_all(), slots, st["dtype"])
    ver = oracle.greedy_verify(r["logits"], "f32", r["drafts"])
    return ver


@pytest.mark.parametrize("alpha", [0.2, 0.9, 1.0])
def test_draft_resync_keeps_the_accepted_prefix(alpha):
    """[Design] KV Cache Synchronization: after re-sync the draft cache holds
    the accepted prefix; after full acceptance it lacks only d_k (lag 1)."""
    st = _state(B=6, k=4, rounds=2, seed=int(alpha * 10))
    ver = _draft_round(st, alpha)
    e = ver["emit_count"]
    out = oracle.resync_draft(st["kv"], st["E"], st["model"].n_all(), e, st["k"])
    assert out["ok"]
    assert np.array_equal(out["kept"], np.minimum(e, st["k"]))
    st["model"].commit(ver["out_tokens"], e)
    lag = (e == st["k"] + 1).astype(np.int64)
    if alpha == 1.0:
        assert lag.all()
    assert st["model"].check(out["kv"], out["pos"], out["mask"], out["E_new"], _content("bf16"), lag=lag) == []


def test_draft_resync_equals_target_commit_when_no_sequence_accepts_all():
    st = _state(B=5, k=3, rounds=2, seed=3)
    _draft_round(st, 0.5)
    e = np.array([1, 3, 2, 3, 1])                       # every e <= k
    a = oracle.resync_draft(st["kv"], st["E"], st["model"].n_all(), e, st["k"])
    b = oracle.commit_realign(st["kv"], st["E"], st["model"].n_all(), e, st["k"])
    for key in ["kv", "pos", "mask", "E_new", "kv_len", "bytes_moved"]:
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key


def test_negative_control_draft_keeps_an_unwritten_slot():
    """Keeping k + 1 draft slots after full acceptance keeps a column the draft
    never wrote; the invariant check catches it."""
    st = _state(B=4, k=3, rounds=2, seed=5)
    ver = _draft_round(st, 1.0)
    e = ver["emit_count"]
    wrong = oracle.commit_realign(st["kv"], st["E"], st["model"].n_all(), e, st["k"])
    st["model"].commit(ver["out_tokens"], e)
    assert st["model"].check(wrong["kv"], None, None, wrong["E_new"], _content("bf16"))


def test_draft_resync_capacity_and_bad_state():
    st = _state(B=3, k=3, rounds=1, seed=6)
    n = st["model"].n_all()
    C = st["E"] + st["k"]                              # room for exactly k draft slots
    ok = oracle.resync_draft(st["kv"][:, :, :, :, :C], st["E"], n, [1, 2, 3], st["k"])
    assert ok["ok"]
    bad = oracle.resync_draft(st["kv"][:, :, :, :, :C - 1], st["E"], n, [1, 2, 3], st["k"])
    assert not bad["ok"] and (bad["status"] & oracle.ST_CAPACITY).all()
    bad = oracle.resync_draft(st["kv"], st["E"], n, [1, 5, 3], st["k"])
    assert not bad["ok"] and bad["status"][1] & oracle.ST_BAD_STATE
