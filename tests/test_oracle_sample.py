"""Pins for the stochastic oracle: worked examples by exact enumeration,
output-count law, Monte Carlo, residual identity, negative controls."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.sample as osample
from workloads import sample_round


def _frac(xs):
    return [Fraction(x) for x in xs]


def _enumerate(p_str, q_str, k, N=10, eos_id=-1, remaining=None):
    """Exact outcome law of sample_verify over every draft tuple (weight prod q)
    and a stratified grid of uniforms u = (i + 1/2) / N for each of the k+1 draws.

    Returns (law of emitted token lists as {tuple: Fraction}).
    """
    V = len(p_str)
    p = np.array([float(x) for x in p_str], np.float32)
    q = np.array([float(x) for x in q_str], np.float32)
    qf = _frac(q_str)
    grid = [(i + 0.5) / N for i in range(N)]
    drafts, unis, weights = [], [], []
    for xs in itertools.product(range(V), repeat=k):
        w = Fraction(1)
        for x in xs:
            w *= qf[x]
        if w == 0:
            continue
        for us in itertools.product(range(N), repeat=k + 1):
            drafts.append(xs)
            unis.append([grid[i] for i in us])
            weights.append(w / N ** (k + 1))
    B = len(drafts)
    P = np.broadcast_to(p, (B, k + 1, V)).copy()
    Q = np.broadcast_to(q, (B, k, V)).copy()
    res = oracle.sample_verify(P, Q, np.array(drafts, np.int32), np.array(unis, np.float32),
                               eos_id=eos_id, remaining=remaining)
    law = {}
    for b in range(B):
        key = tuple(int(t) for t in res["out_tokens"][b, :res["emit_count"][b]])
        law[key] = law.get(key, Fraction(0)) + weights[b]
    return law


def _slot_law(law, slot, V):
    """P(token at `slot` = v | at least slot+1 tokens emitted)."""
    reach = sum(w for toks, w in law.items() if len(toks) > slot)
    return [sum(w for toks, w in law.items() if len(toks) > slot and toks[slot] == v) / reach
            for v in range(V)]


def test_two_symbol_example_exact(load_golden):
    g = load_golden("stochastic_two_symbol.json")
    law = _enumerate(g["p"], g["q"], k=1)
    assert _slot_law(law, 0, 2) == _frac(g["output_distribution"])
    # acceptance probabilities as printed
    for x, want in enumerate(_frac(g["accept_probability"])):
        a, st = oracle.accept_probability(np.float32(float(g["p"][x])), np.float32(float(g["q"][x])))
        assert Fraction(float(a)).limit_denominator(1000) == want and st == 0


def test_three_symbol_example_exact(load_golden):
    g = load_golden("stochastic_three_symbol.json")
    V = 3
    p, q = g["p"], g["q"]
    for x, want in enumerate(_frac(g["accept_probability"])):
        a, _ = oracle.accept_probability(np.float32(float(p[x])), np.float32(float(q[x])))
        assert Fraction(float(a)).limit_denominator(1000) == want
    # accepted mass min(p, q) and alpha
    acc = [min(a, b) for a, b in zip(_frac(p), _frac(q))]
    assert acc == _frac(g["accepted_mass"]) and sum(acc) == Fraction(g["alpha"])
    # residual normalises to [1, 0, 0]: every draw from it is token 0
    resid = osample._residual(np.array([float(x) for x in p], np.float32),
                              np.array([float(x) for x in q], np.float32))
    for u in np.linspace(0, 0.999, 37, dtype=np.float32):
        assert oracle.draw_from_mass(resid, u)[0] == 0
    # one proposal: output law is p exactly
    law1 = _enumerate(p, q, k=1)
    assert _slot_law(law1, 0, V) == _frac(g["output_distribution"])
    # two iid proposals: every emitted slot is p-distributed, and the count
    # law is 0.4 / 0.24 / 0.36 with mean 1.96
    law2 = _enumerate(p, q, k=2)
    for slot in range(3):
        assert _slot_law(law2, slot, V) == _frac(g["output_distribution"])
    count = {n: sum(w for t, w in law2.items() if len(t) == n) for n in (1, 2, 3)}
    assert count == {int(n): Fraction(v) for n, v in g["output_count_distribution"].items()}
    assert sum(n * w for n, w in count.items()) == Fraction(g["expected_output_count"])


def test_negative_control_resample_from_p(monkeypatch, load_golden):
    g = load_golden("stochastic_two_symbol.json")
    monkeypatch.setattr(osample, "_residual", lambda p_row, q_row: p_row.copy())
    law = _enumerate(g["p"], g["q"], k=1)
    got = _slot_law(law, 0, 2)
    assert got != _frac(g["output_distribution"])
    assert got == _frac(g["wrong_resample_from_p_output"])


def test_negative_control_bonus_from_draft(monkeypatch, load_golden):
    """Taking the bonus from the draft distribution (the bug class the
    forensics paper reports for one prior system) breaks the output law."""
    g = load_golden("stochastic_three_symbol.json")
    qrow = np.array([float(x) for x in g["q"]], np.float32)
    monkeypatch.setattr(osample, "_bonus_row", lambda p, b, k: qrow)
    law = _enumerate(g["p"], g["q"], k=1)
    assert _slot_law(law, 1, 3) != _frac(g["output_distribution"])


def test_output_count_monte_carlo(load_golden):
    g = load_golden("stochastic_three_symbol.json")
    k = g["iid_gamma"]
    p = np.array([float(x) for x in g["p"]], np.float32)
    q = np.array([float(x) for x in g["q"]], np.float32)
    B = 200_000
    rng = np.random.default_rng(123)
    drafts = rng.choice(3, size=(B, k), p=q.astype(np.float64) / q.sum()).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    res = oracle.sample_verify(np.broadcast_to(p, (B, k + 1, 3)).copy(),
                               np.broadcast_to(q, (B, k, 3)).copy(), drafts, u)
    K = res["emit_count"].astype(np.float64)
    mean = float(g["expected_output_count"])
    law = np.array([float(v) for v in g["output_count_distribution"].values()])
    var = float((law * np.array([1, 4, 9])).sum() - mean ** 2)   # 0.7584
    assert abs(K.mean() - mean) < 5 * math.sqrt(var / B)
    freq = np.bincount(res["emit_count"], minlength=4)[1:] / B
    assert np.allclose(freq, law, atol=5 * math.sqrt(0.25 / B))
    # the correction is always token 0 in this toy (residual [1, 0, 0])
    rejected = res["emit_count"] - res["accept_len"] == 1
    rejected &= res["emit_count"] <= k
    last = res["out_tokens"][np.arange(B), res["emit_count"] - 1]
    assert (last[rejected] == 0).all()


def test_residual_mass_identity():
    """sum max(p - q, 0) = 1 - alpha, alpha = sum min(p, q), for normalised rows."""
    r = sample_round(2, B=2, V=5000)
    for b in range(2):
        for j in range(r["k"]):
            pj, qj = r["p"][b, j], r["q"][b, j]
            _, S = oracle.draw_from_mass(osample._residual(pj, qj), 0.5)
            alpha = math.fsum(np.minimum(pj, qj).astype(np.float64))
            assert abs(S - (math.fsum(pj.astype(np.float64)) - alpha)) < 1e-6
            assert 0.0 < S < 1.0


@pytest.mark.parametrize("px,qx,want,st", [
    (0.3, 0.6, 0.5, 0), (0.6, 0.2, 1.0, 0), (0.25, 0.25, 1.0, 0),
    (0.2, 0.0, 1.0, oracle.ST_Q_ZERO), (0.0, 0.0, 0.0, oracle.ST_Q_ZERO),
])
def test_accept_probability_cases(px, qx, want, st):
    a, s = oracle.accept_probability(np.float32(px), np.float32(qx))
    assert a == np.float32(want) and s == st


def test_accept_probability_is_one_float32_division():
    """The ratio is the correctly rounded float32 quotient.  A float64 quotient
    of two float32 values rounded once more to float32 is correctly rounded
    (float64 carries more than 2*24+2 bits), which gives an independent value."""
    rng = np.random.default_rng(5)
    px = rng.random(5000).astype(np.float32)
    qx = rng.random(5000).astype(np.float32) + np.float32(1e-3)
    for a, b in zip(px, qx):
        got, _ = oracle.accept_probability(a, b)
        want = np.float32(np.float64(a) / np.float64(b))
        assert got == min(np.float32(1.0), want)


def test_draw_never_picks_zero_mass():
    r = np.array([0.2, 0.0, 0.8], np.float32)
    assert oracle.draw_from_mass(r, np.float32(0.0))[0] == 0
    assert oracle.draw_from_mass(r, np.float32(0.25))[0] == 2
    assert oracle.draw_from_mass(np.array([0, 1, 0], np.float32), np.float32(0.9999))[0] == 1
    assert oracle.draw_from_mass(np.zeros(3, np.float32), np.float32(0.5))[0] is None


def test_zero_residual_falls_back_to_p():
    # unnormalised rows with p < q everywhere: rejection leaves no residual
    p = np.array([[[0.1, 0.1], [0.1, 0.1]]], np.float32)
    q = np.array([[[0.5, 0.5]]], np.float32)
    res = oracle.sample_verify(p, q, np.array([[1]], np.int32), np.array([[0.9, 0.75]], np.float32))
    assert res["status"][0] == oracle.ST_RESID_ZERO
    assert res["out_tokens"][0].tolist() == [1, -1]           # 0.75 * 0.2 lands in token 1
    assert abs(res["final_mass"][0] - float(np.float32(0.1)) * 2) < 1e-9


def test_out_of_range_draft_is_rejected():
    p = np.array([[[0.5, 0.5], [0.5, 0.5]]], np.float32)
    q = np.array([[[0.5, 0.5]]], np.float32)
    res = oracle.sample_verify(p, q, np.array([[7]], np.int32), np.array([[0.0, 0.1]], np.float32))
    # p == q leaves no residual, so the correction falls back to p as well
    assert res["status"][0] == oracle.ST_DRAFT_OOR | oracle.ST_RESID_ZERO
    assert res["accept_len"][0] == 0 and res["emit_count"][0] == 1


def test_eos_and_budget_stop_without_draw():
    V, k = 4, 3
    p = np.full((1, k + 1, V), 0.25, np.float32)
    q = np.full((1, k, V), 0.25, np.float32)      # p == q: always accepted
    d = np.array([[2, 3, 1]], np.int32)
    u = np.array([[0.5, 0.5, 0.5, 0.5]], np.float32)
    assert oracle.sample_verify(p, q, d, u, eos_id=3)["out_tokens"][0].tolist() == [2, 3, -1, -1]
    r2 = oracle.sample_verify(p, q, d, u, remaining=np.array([2]))
    assert r2["out_tokens"][0].tolist() == [2, 3, -1, -1] and r2["final_mass"][0] == 0.0
    r0 = oracle.sample_verify(p, q, d, u, remaining=np.array([0]))
    assert r0["emit_count"][0] == 0
    full = oracle.sample_verify(p, q, d, u)
    assert full["emit_count"][0] == 4 and full["out_tokens"][0, 3] == 2   # bonus: 0.5 of 4 -> id 2
