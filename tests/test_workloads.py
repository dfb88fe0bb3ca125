"""The seeded generators: determinism, shapes, numpy/torch agreement."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    x[:6] = [0.0, -0.0, 1.0, -2.5, 3.0e38, 1.0e-30]
    ours = W.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_streams_deterministic_and_independent():
    a = W.stream(3, "logits", 2).random(8)
    b = W.stream(3, "logits", 2).random(8)
    c = W.stream(3, "logits", 3).random(8)
    d = W.stream(3, "drafts", 2).random(8)
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)


@pytest.mark.parametrize("c", [0, 1])
def test_greedy_round_shapes_and_planting(c):
    cfg = W.workload(c)
    r = W.greedy_round(c)
    B, k, V = cfg["B"], cfg["k"], cfg["V"]
    assert r["logits"].shape == (B, k + 1, V)
    assert r["logits"].dtype == (np.uint16 if cfg["logit_dtype"] == "bf16" else np.float32)
    assert r["drafts"].shape == (B, k) and r["drafts"].dtype == np.int32
    assert ((r["drafts"] >= 0) & (r["drafts"] < V)).all()
    r2 = W.greedy_round(c)
    assert np.array_equal(r["logits"], r2["logits"]) and np.array_equal(r["drafts"], r2["drafts"])


def test_sample_round_is_distribution():
    r = W.sample_round(2, B=2, V=4096)
    assert r["p"].shape == (2, 5, 4096) and r["q"].shape == (2, 4, 4096)
    assert np.allclose(r["p"].astype(np.float64).sum(-1), 1, atol=1e-5)
    assert (r["q"] > 0).all() and (r["uniforms"] >= 0).all() and (r["uniforms"] < 1).all()
    assert r["uniforms"].dtype == np.float32


def test_geometry_and_pool():
    for c in range(4):
        g = W.kv_geometry(c, rounds=3)
        cfg = W.workload(c)
        lo, hi = cfg["prefix"]
        assert (g["n"] >= lo - 1).all() and (g["n"] <= hi - 1).all()
        assert g["E"] == g["n"].max() and g["C"] == g["E"] + 3 * (cfg["k"] + 1)
    P = W.pool_lengths()
    assert P.shape == (256,) and (P >= 64 + 8).all() and (P <= 2048 + 8 * 5).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_fill_numpy_torch_agree(dtype):
    B, L, H, D, k = 3, 2, 3, 16, 4
    n = np.array([5, 9, 0])
    E = 9
    C = E + k + 1 + 3
    toks = np.random.default_rng(1).integers(0, 100, size=(B, 10))
    a = W.fill_kv_np(L, H, D, B, C, E, n, toks, dtype)
    slots = np.random.default_rng(2).integers(0, 100, size=(B, k + 1))
    W.write_forward_slots_np(a, E, n, slots, dtype)
    t = torch.empty(a.shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    W.fill_kv_torch(t, E, n, torch.as_tensor(toks), dtype)
    W.write_forward_slots_torch(t, E, n, torch.as_tensor(slots), dtype)
    iv = t.view(torch.int16 if dtype == "bf16" else torch.int32).numpy().view(a.dtype)
    assert np.array_equal(iv, a)
    vals = t.float().numpy()
    assert np.isfinite(vals).all() and (vals != 0).all()


def test_accept_counts_follow_the_planted_law():
    """Synthetic emitted counts: mean over rounds equals (1 - a^(k+1)) / (1 - a)."""
    import workloads as W
    k = W.workload(3)["k"]
    a = W.alphas(3)
    e = np.stack([W.accept_counts(3, r) for r in range(4000)])
    assert e.min() >= 1 and e.max() <= k + 1
    want = (1 - a ** (k + 1)) / (1 - a)
    se = e.std(axis=0) / np.sqrt(e.shape[0])
    assert np.all(np.abs(e.mean(axis=0) - want) < 5 * se + 1e-9)
    assert np.array_equal(W.accept_counts(3, 7, B=5), W.accept_counts(3, 7)[:5])
