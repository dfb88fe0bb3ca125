"""Pins for the processed-distribution oracle (temperature, top-k, top-p).

The pages only require that p and q be the processed distributions
([Walkthrough] 5.1); the operations follow their usual definitions.  The pins
tie the oracle to things other than itself: a library softmax, the closed
form of temperature scaling, hand-derived worked examples (tests/golden),
brute force over tiny inputs, and the exact output law of the verification
run on processed rows.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle.process import process_row, process_rows, sample_verify_logits


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def test_plain_softmax_is_the_library_routine():
    rng = np.random.default_rng(1)
    z = (rng.standard_normal(5000) * 3).astype(np.float32)
    p, info = process_row(z, 1.0)
    ref = softmax(z.astype(np.float64)).astype(np.float32)
    assert _ulps(p, ref).max() <= 1
    assert info["kept"].all()


@pytest.mark.parametrize("T", [0.25, 0.5, 0.7, 2.0])
def test_temperature_closed_form(T):
    """softmax(z / T) is proportional to softmax(z) ** (1 / T)."""
    rng = np.random.default_rng(2)
    z = (rng.standard_normal(300) * 2).astype(np.float32)
    p, _ = process_row(z, T)
    base = softmax(z.astype(np.float64))
    ref = base ** (1.0 / float(np.float32(T)))
    ref /= ref.sum()
    assert np.allclose(p, ref, rtol=2e-6, atol=1e-30)


def test_top_k_one_is_the_argmax_and_ties_share():
    z = np.array([0.5, 2.0, -1.0, 1.5], np.float32)
    p, _ = process_row(z, 0.9, top_k=1)
    assert p.tolist() == [0.0, 1.0, 0.0, 0.0]
    z = np.array([2.0, 0.5, 2.0, 1.0], np.float32)          # tie at the boundary: both kept
    p, info = process_row(z, 1.0, top_k=1)
    assert p.tolist() == [0.5, 0.0, 0.5, 0.0]
    assert info["kept"].sum() == 2


def test_top_k_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 12))
        z = rng.integers(-3, 4, size=V).astype(np.float32)  # many repeats
        K = int(rng.integers(0, V + 2))
        _, info = process_row(z, 1.3, top_k=K)
        if K == 0 or K >= V:
            ref = np.ones(V, bool)
        else:
            ranked = sorted(z.tolist(), reverse=True)
            ref = z >= ranked[K - 1]
        assert np.array_equal(info["kept"], ref)
        assert info["kept"].sum() >= min(max(K, 1), V) if K else True


def _brute_top_p(z, T, top_p):
    """Smallest top set by logit (whole tie groups) whose mass reaches top_p."""
    z64 = z.astype(np.float64)
    w = np.exp((z64 - z64.max()) / float(np.float32(T)))
    total = math.fsum(w)
    vals = sorted(set(z64.tolist()), reverse=True)
    for n in range(1, len(vals) + 1):
        keep = z64 >= vals[n - 1]
        above = math.fsum(w[z64 > vals[n - 1]])
        nxt_above = math.fsum(w[keep])
        if n == len(vals) or nxt_above >= float(np.float32(top_p)) * total:
            assert above < float(np.float32(top_p)) * total or n == 1
            return keep
    raise AssertionError


def test_top_p_brute_force():
    rng = np.random.default_rng(4)
    for _ in range(300):
        V = int(rng.integers(1, 10))
        z = (rng.integers(-4, 5, size=V) * 0.5).astype(np.float32)
        top_p = float(rng.choice([0.1, 0.3, 0.5, 0.77, 0.9, 0.99]))
        T = float(rng.choice([0.5, 1.0, 1.7]))
        _, info = process_row(z, T, top_p=top_p)
        assert np.array_equal(info["kept"], _brute_top_p(z, T, top_p)), (z, T, top_p)


def test_worked_examples(load_golden):
    g = load_golden("processed_distributions.json")
    for case in g["cases"]:
        z = np.log(np.array(case["probs"], np.float64)).astype(np.float32)
        p, info = process_row(z, 1.0, top_k=case.get("top_k", 0), top_p=case.get("top_p", 1.0))
        want = np.array([float(Fraction(x)) for x in case["expect"]], np.float64)
        assert np.allclose(p, want, rtol=1e-6, atol=0), (case["name"], p, want)
        assert info["kept"].sum() == case["kept"], case["name"]


def test_rows_of_minus_infinity_and_masked_entries():
    z = np.array([-np.inf, -np.inf, -np.inf], np.float32)
    p, info = process_row(z, 1.0, top_k=2, top_p=0.5)
    assert p.tolist() == [0.0, 0.0, 0.0] and info["mass"] == 0.0
    z = np.array([-np.inf, 1.0, -np.inf, 1.0], np.float32)
    p, _ = process_row(z, 0.8, top_p=0.9)
    assert p.tolist() == [0.0, 0.5, 0.0, 0.5]


def test_processed_verification_reproduces_the_processed_target():
    """Output law of the verification on processed rows is p' (drafts weighted
    by q', stratified uniform grids for the acceptance and the draw)."""
    zp = np.log(np.array([0.5, 0.3, 0.15, 0.05])).astype(np.float32)
    zq = np.log(np.array([0.1, 0.2, 0.3, 0.4])).astype(np.float32)
    T, K, top_p = 0.8, 3, 0.95
    p1, _ = process_row(zp, T, K, top_p)
    q1, _ = process_row(zq, T, K, top_p)
    V, k, N = 4, 1, 250
    grid = np.array([(i + 0.5) / N for i in range(N)], np.float32)
    xs = [x for x in range(V) if q1[x] > 0]
    X, A, D = np.meshgrid(np.array(xs), grid, grid, indexing="ij")
    drafts = X.reshape(-1, 1).astype(np.int32)
    unis = np.stack([A.reshape(-1), D.reshape(-1)], axis=1).astype(np.float32)
    wts = q1[drafts[:, 0]].astype(np.float64) / (N * N)
    B = drafts.shape[0]
    P = np.broadcast_to(p1, (B, k + 1, V)).copy()
    Q = np.broadcast_to(q1, (B, k, V)).copy()
    out = oracle.sample_verify(P, Q, drafts, unis)
    law = np.bincount(out["out_tokens"][:, 0], weights=wts, minlength=V)
    assert np.allclose(law, p1, atol=2e-3)
    # the composed entry point equals processing followed by verification
    small = slice(0, 7)
    ZP = np.broadcast_to(zp, (7, k + 1, V)).copy()
    ZQ = np.broadcast_to(zq, (7, k, V)).copy()
    a = sample_verify_logits(ZP, ZQ, drafts[small], unis[small], T, K, top_p)
    b = oracle.sample_verify(P[small], Q[small], drafts[small], unis[small])
    for key in a:
        assert np.array_equal(a[key], b[key])


def test_processing_matches_stochastic_oracle_on_given_rows():
    """With no truncation and T = 1, processing softmax logits reproduces the
    given probabilities, so the processed verification equals the plain one."""
    rng = np.random.default_rng(5)
    B, k, V = 6, 3, 40
    p = softmax(rng.standard_normal((B, k + 1, V)), axis=-1)
    q = softmax(rng.standard_normal((B, k, V)), axis=-1)
    zp, zq = np.log(p).astype(np.float32), np.log(q).astype(np.float32)
    pp, _ = process_rows(zp, 1.0)
    qq, _ = process_rows(zq, 1.0)
    d = rng.integers(0, V, size=(B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    a = sample_verify_logits(zp, zq, d, u, 1.0)
    b = oracle.sample_verify(pp, qq, d, u)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert np.allclose(pp, p, rtol=3e-6)
