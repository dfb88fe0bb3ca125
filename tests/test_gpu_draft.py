"""GPU parity of the draft-cache re-sync (spec_resync_draft_kv) against the
oracle: the moved KV bytes, lengths, end column, byte count and (optional)
positions and mask must equal the oracle's exactly, and a target + draft round
must leave both caches in the state per-sequence decoding implies."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import (DEV, commit, host, i32, kv_bits, logits_to_device, note, requires_gpu, resync,
                        verify_greedy)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _cache(L, H, D, B, C, E, n, tokens, dt):
    kv = torch.empty((L, 2, B, H, C, D), dtype=_tdt(dt), device=DEV)
    W.fill_kv_torch(kv, E, n, torch.as_tensor(tokens).to(DEV), dt)
    return kv


def _check(kv, k, E, n, e, pos_mask=True):
    pre = kv_bits(kv)
    ref = oracle.resync_draft(pre, E, n, e, k)
    got = host(resync(kv, k, E, n, e, pos_mask))
    assert ref["ok"]
    assert np.array_equal(kv_bits(kv), ref["kv"])
    if pos_mask:
        assert np.array_equal(got["pos"], ref["pos"]) and np.array_equal(got["mask"], ref["mask"])
    assert np.array_equal(got["kv_len"], ref["kv_len"])
    assert int(got["end_col"][0]) == ref["E_new"]
    assert int(got["bytes_moved"][0]) == ref["bytes_moved"]
    assert (got["status"] == 0).all()


def test_resync_random_stress():
    rng = np.random.default_rng(21)
    for it in range(50):
        dt = "bf16" if it % 2 else "f32"
        L, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        D = int(rng.choice([1, 3, 8, 64, 128]))
        B, k = int(rng.integers(1, 9)), int(rng.integers(1, 12))
        n = rng.integers(0, 300, B)
        E = int(n.max()) + int(rng.integers(0, 5))
        C = E + k + int(rng.integers(0, 5))               # room for the k draft slots
        e = rng.integers(0, k + 2, B)
        note(f"resync stress {it}: L={L} H={H} D={D} B={B} k={k} E={E} C={C} {dt}")
        kv = _cache(L, H, D, B, C, E, n, rng.integers(0, 99, (B, E + 1)), dt)
        _check(kv, k, E, n, e, pos_mask=bool(it % 3))


def test_resync_full_acceptance_and_uniform_cases():
    rng = np.random.default_rng(22)
    L, H, D, B, k = 2, 2, 64, 5, 4
    n = np.array([10, 3, 0, 25, 7])
    E, C = 26, 30
    for e in ([5, 5, 5, 5, 5], [4, 5, 1, 5, 0], [2, 2, 2, 2, 2], [4, 4, 4, 4, 5]):
        note(f"resync cases e={e}")
        kv = _cache(L, H, D, B, C, E, n, rng.integers(0, 50, (B, E + 1)), "bf16")
        _check(kv, k, E, n, np.array(e))


def test_resync_capacity_changes_nothing():
    rng = np.random.default_rng(23)
    L, H, D, B, k = 1, 2, 8, 3, 4
    n = np.array([5, 2, 6])
    E, C = 6, 9                                          # E + k > C
    kv = _cache(L, H, D, B, C, E, n, rng.integers(0, 50, (B, E + 1)), "f32")
    before = kv_bits(kv)
    note("resync capacity")
    got = host(resync(kv, k, E, n, np.array([1, 2, 3])))
    assert np.array_equal(kv_bits(kv), before)
    assert (got["status"] & oracle.ST_CAPACITY).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_target_and_draft_rounds(dt):
    """Each round: the target forward writes k+1 slots, the draft forward k;
    verification on the GPU; target commit and draft re-sync on the GPU.  Both
    caches must match per-sequence decoding (the draft lags one entry after a
    full acceptance).  The draft cache is re-seeded from the committed tokens
    whenever it lags, as a drafting step that catches up would."""
    rng = np.random.default_rng(24)
    L, H, D, B, k, V, R = 2, 2, 32, 6, 4, 300, 12
    P = rng.integers(2, 30, B)
    toks = [rng.integers(0, V, int(p)).tolist() for p in P]
    model = oracle.UnbatchedModel(toks)
    content = lambda b, pos, tok, plane, d: W.kv_bits_np(b, pos, tok, plane, d, dt)
    for r in range(R):
        n = model.n_all()
        E = int(n.max())
        C = E + k + 1
        grid = np.zeros((B, E + 2), np.int64)
        for b in range(B):
            grid[b, :len(model.tokens[b])] = model.tokens[b]
        tkv = _cache(L, H, D, B, C, E, n, grid, dt)
        dkv = _cache(L, H, D, B, C, E, n, grid, dt)
        g = W.planted_greedy(rng, rng, B, k, V, 1.0, "f32", rng.uniform(0.3, 1.0, B))
        slots = model.slot_tokens(g["drafts"])
        W.write_forward_slots_torch(tkv, E, n, torch.as_tensor(slots).to(DEV), dt)
        W.write_forward_slots_torch(dkv, E, n, torch.as_tensor(slots[:, :k]).to(DEV), dt)
        note(f"target+draft round {r} {dt}")
        gv = verify_greedy(logits_to_device(g["logits"], "f32"), g["drafts"])
        ct = host(commit(tkv, k, E, n, gv["emit_count"]))
        cd = host(resync(dkv, k, E, n, gv["emit_count"]))
        e = host(gv)["emit_count"]
        ver = oracle.greedy_verify(g["logits"], "f32", g["drafts"])
        assert np.array_equal(e, ver["emit_count"])
        model.commit(ver["out_tokens"], e)
        assert model.check(kv_bits(tkv), ct["pos"], ct["mask"], int(ct["end_col"][0]), content) == []
        lag = (e == k + 1).astype(np.int64)
        assert model.check(kv_bits(dkv), cd["pos"], cd["mask"], int(cd["end_col"][0]), content, lag=lag) == []
        assert np.array_equal(cd["kv_len"], ct["kv_len"] - lag)
