"""Pins for the greedy oracle: worked example, row alignment, tie rule,
stopping rules, closed-form expected output count."""
import numpy as np
import pytest

import oracle
from workloads import planted_greedy, bf16_bits_from_f32


def _rows_with_argmax(choices, V, rng):
    """Rows whose unique maximum sits at the given indices."""
    rows = rng.standard_normal((len(choices), V)).astype(np.float32)
    for i, c in enumerate(choices):
        rows[i, c] = rows[i].max() + 1.0
    return rows


def test_worked_rejection(load_golden):
    g = load_golden("greedy_worked_rejection.json")
    rng = np.random.default_rng(0)
    V = 8
    # rows 2 and 3 are discarded by the rule; give them arbitrary maxima
    rows = _rows_with_argmax(g["target_argmax_first_rows"] + [5, 6], V, rng)
    toks, acc = oracle.greedy_commit(rows, g["drafts"])
    assert toks == g["commit"]
    assert acc == g["accepted"]
    # batched form agrees and pads with -1
    res = oracle.greedy_verify(rows[None], "f32", np.array([g["drafts"]], np.int32))
    assert res["out_tokens"][0].tolist() == g["commit"] + [-1, -1]
    assert res["emit_count"][0] == 2 and res["accept_len"][0] == 1
    assert res["emit_offsets"].tolist() == [0, 2]


def test_row_alignment_exercise(load_golden):
    g = load_golden("row_alignment_exercise.json")
    L, k = g["prefix_len"], g["k"]
    V = 32
    # a full-prefix forward over L + k inputs; row i's argmax encodes i
    full = np.zeros((L + k, V), np.float32)
    for i in range(L + k):
        full[i, i] = 1.0
    rows = oracle.verification_rows(full, L)
    assert rows.shape[0] == k + 1
    got = [oracle.argmax_first(r) for r in rows]
    assert got[:k] == g["verify_rows"]
    assert got[k] == g["bonus_row"]


@pytest.mark.parametrize("row,want", [
    ([0.0, 3.0, 1.0, 3.0], 1),            # tie: lowest index
    ([-0.0, 0.0, -1.0], 0),               # -0 == +0
    ([0.0, -0.0], 0),
    ([-1.0, -0.0, 0.0, -0.0], 1),
    ([-np.inf, -np.inf, -np.inf], 0),     # all -inf: index 0
    ([-np.inf, -5.0, -np.inf], 1),
    ([np.inf, 1.0, np.inf], 0),
    ([7.0], 0),
])
def test_argmax_tie_rule(row, want):
    assert oracle.argmax_first(np.array(row, np.float32)) == want


def test_argmax_bruteforce_tiny():
    # every row over {-1, -0, +0, 1, 2} of length 3: the winner is the first
    # position whose value is not exceeded by any other position
    vals = [-1.0, -0.0, 0.0, 1.0, 2.0]
    import itertools
    for row in itertools.product(vals, repeat=3):
        r = np.array(row, np.float32)
        want = next(i for i in range(3) if all(not (r[j] > r[i]) for j in range(3)))
        assert oracle.argmax_first(r) == want


def test_bf16_widening_exact_and_ties():
    x = np.array([1.0, 2.0, -3.5, 0.0, -0.0, 65280.0, 2.0 ** -126, -np.inf], np.float32)
    bits = bf16_bits_from_f32(x)
    assert np.array_equal(oracle.widen_bf16(bits), x)
    # bf16 ties across the row resolve to the first index
    row = bf16_bits_from_f32(np.array([0.5, 2.0, 2.0, 1.0], np.float32))
    res = oracle.greedy_verify(np.stack([row, row])[None], "bf16", np.array([[9]], np.int32))
    assert res["out_tokens"][0].tolist() == [1, -1]
    assert res["status"][0] == oracle.ST_DRAFT_OOR  # 9 >= V=4


def _budget_case(k=3, V=10):
    rng = np.random.default_rng(1)
    choices = [3, 4, 5, 6]
    return _rows_with_argmax(choices, V, rng), choices


@pytest.mark.parametrize("budget,want", [
    (0, []), (1, [3]), (2, [3, 4]), (3, [3, 4, 5]), (4, [3, 4, 5, 6]), (9, [3, 4, 5, 6]),
])
def test_output_budget(budget, want):
    rows, choices = _budget_case()
    toks, acc = oracle.greedy_commit(rows, choices[:3], remaining=budget)
    assert toks == want
    assert acc == min(len(want), 3)


def test_eos_proposed_and_matched_stops():
    rows, choices = _budget_case()
    toks, acc = oracle.greedy_commit(rows, choices[:3], eos_id=4)
    assert toks == [3, 4] and acc == 2


def test_eos_proposed_but_rejected_commits_correction():
    # walkthrough exercise 4: a rejected EOS proposal commits the target's
    # correction; the round ends at the mismatch, not at EOS
    rows, choices = _budget_case()
    eos = 8
    toks, acc = oracle.greedy_commit(rows, [3, eos, 5], eos_id=eos)
    assert toks == [3, 4] and acc == 1 and toks[-1] != eos


def test_correction_is_eos():
    rows, choices = _budget_case()
    toks, acc = oracle.greedy_commit(rows, [3, 9, 5], eos_id=4)
    assert toks == [3, 4] and acc == 1


def test_bonus_eos_and_full_acceptance():
    rows, choices = _budget_case()
    toks, acc = oracle.greedy_commit(rows, choices[:3], eos_id=6)
    assert toks == [3, 4, 5, 6] and acc == 3


def test_key_property_extremes(load_golden):
    """All drafts accepted -> k+1 tokens; none accepted -> 1 token equal to
    non-speculative argmax decoding (design document, Key Property)."""
    rng = np.random.default_rng(2)
    B, k, V = 64, 5, 50
    logits = rng.standard_normal((B, k + 1, V)).astype(np.float32)
    best = np.argmax(logits, axis=-1)
    all_ok = oracle.greedy_verify(logits, "f32", best[:, :k].astype(np.int32))
    assert (all_ok["emit_count"] == k + 1).all()
    assert np.array_equal(all_ok["out_tokens"], best)
    wrong = ((best[:, :k] + 1) % V).astype(np.int32)
    none = oracle.greedy_verify(logits, "f32", wrong)
    assert (none["emit_count"] == 1).all() and (none["accept_len"] == 0).all()
    assert np.array_equal(none["out_tokens"][:, 0], best[:, 0])


def test_expected_output_count_monte_carlo(load_golden):
    """Planted iid acceptance alpha: mean emitted per round = (1-a^(k+1))/(1-a)."""
    g = load_golden("expected_tokens_per_step.json")
    case = next(c for c in g["cases"] if c["gamma"] == 4)
    a, k = float(case["alpha"]), case["gamma"]
    closed = (1 - a ** (k + 1)) / (1 - a)
    assert abs(closed - float(case["expected"])) < 1e-5
    B, V = 40000, 16
    r = planted_greedy(np.random.default_rng(10), np.random.default_rng(11), B, k, V, 1.0, "f32", a)
    res = oracle.greedy_verify(r["logits"], "f32", r["drafts"])
    e = res["emit_count"].astype(np.float64)
    # exact variance of the truncated geometric count
    pk = np.array([a ** (j - 1) * (1 - a) for j in range(1, k + 1)] + [a ** k])
    js = np.arange(1, k + 2)
    var = (pk * js ** 2).sum() - closed ** 2
    assert abs(e.mean() - closed) < 5 * np.sqrt(var / B)
    # and the empirical count distribution matches the truncated geometric law
    hist = np.bincount(res["emit_count"], minlength=k + 2)[1:] / B
    assert np.allclose(hist, pk, atol=5 * np.sqrt(0.25 / B))
