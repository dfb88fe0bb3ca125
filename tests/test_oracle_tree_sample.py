"""Pins of the stochastic tree oracle (oracle/tree_sample.py) by what the
method fixes rather than by retyping it:

  * a chain tree is the linear stochastic verification, whose own pins are the
    pages' worked examples (oracle/sample.py, tests/test_oracle_sample.py);
  * distribution preservation ([Atlas] "Acceptance and rejection correction":
    the verified output follows the target): with the children of a node
    drawn independently from the draft distribution at that node, every
    emitted token follows the target's row at its node.  Checked exactly by
    enumerating every draft tuple (weights: products of q as fractions) and a
    stratified grid of uniforms, on toys whose probabilities put every
    decision boundary between grid points; a planted mistake (siblings tried
    against the unreduced target) breaks the law;
  * a Monte Carlo run on a bushier tree over a larger vocabulary;
  * links, budgets, EOS, out-of-range drafts and degenerate residuals."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.tree_sample as ots
from oracle.tree import chain_links


def _links(children, N):
    """first_child / next_sibling [1, N] from {node: [children in order]}."""
    fc = np.full((1, N), -1, np.int32)
    ns = np.full((1, N), -1, np.int32)
    for parent, kids in children.items():
        if kids:
            fc[0, parent] = kids[0]
        for a, b in zip(kids, kids[1:]):
            ns[0, a] = b
    return fc, ns


def _rows(strs):
    return np.array([[float(Fraction(x)) for x in r] for r in strs], np.float32)


def test_chain_is_the_linear_rule():
    """Random chains (k up to 6, V up to 50), with EOS, budgets, out-of-range
    drafts, zero draft probabilities at a proposed token, residuals with no
    mass (p == q) and non-finite entries: every output equal to
    oracle.sample_verify on the same inputs laid out as a linear round."""
    rng = np.random.default_rng(40)
    cases = 0
    for it in range(300):
        B, k, V = int(rng.integers(1, 5)), int(rng.integers(1, 7)), int(rng.integers(2, 50))
        p = rng.dirichlet(np.full(V, 0.5), size=(B, k + 1)).astype(np.float32)
        q = rng.dirichlet(np.full(V, 0.5), size=(B, k)).astype(np.float32)
        if it % 7 == 0:
            q[:, 0] = p[:, 0]                       # residual without mass at the first draft
        d = np.stack([[rng.choice(V, p=q[b, j] / q[b, j].sum()) for j in range(k)] for b in range(B)])
        d = d.astype(np.int32)
        if it % 5 == 0:
            d[0, -1] = V + 3                       # out of range
        if it % 9 == 0 and d[0, 0] < V:
            q[0, 0, d[0, 0]] = 0.0                 # q(x) == 0 at a proposed token
        if it % 11 == 0:
            p[-1, 1, 0] = np.inf
        u = rng.random((B, k + 1)).astype(np.float32)
        eos = int(d[0, 0]) if it % 4 == 1 else -1
        rem = rng.integers(-1, k + 3, B).astype(np.int32) if it % 3 == 2 else None
        lin = oracle.sample_verify(p, q, d, u, eos_id=eos, remaining=rem)
        N = k + 1
        qt = np.concatenate([q, np.zeros((B, 1, V), np.float32)], axis=1)
        dt = np.concatenate([np.zeros((B, 1), np.int32), d], axis=1)
        ut = np.concatenate([u[:, k:], u[:, :k]], axis=1)      # u[b, 0] is the draw
        fc, ns = chain_links(B, N)
        tr = oracle.tree_sample_verify(p, qt, dt, fc, ns, ut, eos_id=eos, remaining=rem)
        for key in ("accept_len", "emit_count", "emit_offsets", "status"):
            assert np.array_equal(tr[key], lin[key]), (it, key)
        assert np.array_equal(tr["out_tokens"][:, :N], lin["out_tokens"]), it
        assert np.array_equal(tr["final_mass"], lin["final_mass"], equal_nan=True), it
        for b in range(B):                         # the kept slots are the chain's first e nodes
            e = int(tr["emit_count"][b])
            assert tr["path"][b, :e].tolist() == list(range(e))
        cases += B
    assert cases > 500


def _enumerate(p, q, fc, ns, draft_parent, grid):
    """Exact law of the emitted token lists: every draft tuple (node c's token
    drawn from q[parent(c)], independently) weighted by the product of those
    q's as fractions, times every point of a stratified grid of the N uniforms.
    p, q: lists of rows of fraction strings, one per node."""
    N, V = len(p), len(p[0])
    pf, qf = _rows(p), _rows(q)
    qfrac = [[Fraction(x) for x in r] for r in q]
    g = [(i + 0.5) / grid for i in range(grid)]
    law = {}
    drafts, unis, weights = [], [], []
    kids = [c for c in range(1, N)]
    for toks in itertools.product(range(V), repeat=len(kids)):
        w = Fraction(1)
        for c, x in zip(kids, toks):
            w *= qfrac[draft_parent[c]][x]
        if w == 0:
            continue
        d = np.zeros(N, np.int32)
        d[1:] = toks
        for us in itertools.product(range(grid), repeat=N):
            drafts.append(d)
            unis.append([g[i] for i in us])
            weights.append(w / grid ** N)
    Bn = len(drafts)
    P = np.broadcast_to(pf, (Bn, N, V)).copy()
    Q = np.broadcast_to(qf, (Bn, N, V)).copy()
    FC = np.broadcast_to(fc, (Bn, N)).copy()
    NS = np.broadcast_to(ns, (Bn, N)).copy()
    r = oracle.tree_sample_verify(P, Q, np.array(drafts), FC, NS, np.array(unis, np.float32))
    assert (r["status"] == 0).all()
    for b in range(Bn):
        key = tuple(int(t) for t in r["out_tokens"][b, :r["emit_count"][b]])
        law[key] = law.get(key, Fraction(0)) + weights[b]
    assert sum(law.values()) == 1
    return law


def _marginal(law, pos, given=None):
    """Law of token `pos` among outcomes that emit it (and whose prefix equals
    `given`), normalised."""
    out, tot = {}, Fraction(0)
    for key, w in law.items():
        if len(key) > pos and (given is None or key[:len(given)] == given):
            out[key[pos]] = out.get(key[pos], Fraction(0)) + w
            tot += w
    return {v: w / tot for v, w in out.items()}, tot


# Root with two leaf children drawn from q0; leaf rows p1.  Tries: a = min(1,
# p0/q0) = (1, 1, 1/3); after one rejection r1 = (3/4, 1/4, 0), a = (1, 1, 0);
# after two r2 = (11/12, 1/12, 0): every boundary is a multiple of 1/12.
P0, Q0, P1 = ["0.5", "0.3", "0.2"], ["0.2", "0.2", "0.6"], ["1/3", "1/4", "5/12"]


def test_two_children_reproduce_the_target_exactly():
    fc, ns = _links({0: [1, 2]}, 3)
    p = [P0, P1, P1]
    q = [Q0, Q0, Q0]
    law = _enumerate(p, q, fc, ns, {1: 0, 2: 0}, grid=12)
    first, _ = _marginal(law, 0)
    assert first == {0: Fraction(1, 2), 1: Fraction(3, 10), 2: Fraction(1, 5)}
    # the token after an accepted child is the bonus from that child's row
    for v in range(3):
        second, tot = _marginal(law, 1, given=(v,))
        if tot:
            assert second == {0: Fraction(1, 3), 1: Fraction(1, 4), 2: Fraction(5, 12)}
    # both children were needed: the second try accepts with positive probability
    r = oracle.tree_sample_verify(_rows([P0, P1, P1])[None], _rows([Q0, Q0, Q0])[None],
                                  np.array([[0, 2, 1]], np.int32), fc, ns,
                                  np.array([[0.5, 0.9, 0.5]], np.float32))
    assert r["out_tokens"][0, 0] == 1 and r["path"][0, :2].tolist() == [0, 2]


def test_two_levels_reproduce_the_target_exactly():
    """Root children 1 and 2 (drawn from q0), node 1's child 3 (drawn from
    q1); rows by depth p0, p1, p2.  Every emitted token follows its depth's
    row: the first p0, the second p1 whatever the first, the third p2."""
    fc, ns = _links({0: [1, 2], 1: [3]}, 4)
    p0, q0 = ["2/3", "1/3"], ["1/3", "2/3"]
    p1, q1, p2 = ["1/3", "2/3"], ["2/3", "1/3"], ["1/2", "1/2"]
    law = _enumerate([p0, p1, p1, p2], [q0, q1, q1, q1], fc, ns, {1: 0, 2: 0, 3: 1}, grid=6)
    first, _ = _marginal(law, 0)
    assert first == {0: Fraction(2, 3), 1: Fraction(1, 3)}
    for v in range(2):
        second, tot = _marginal(law, 1, given=(v,))
        assert tot > 0 and second == {0: Fraction(1, 3), 1: Fraction(2, 3)}
    third, tot = _marginal(law, 2)
    assert tot > 0 and third == {0: Fraction(1, 2), 1: Fraction(1, 2)}


def test_planted_mistake_breaks_the_law(monkeypatch):
    """Trying every sibling against the unreduced target (no residual after a
    rejection) over-produces tokens the draft favours: the exact law fails."""
    def no_reduction(R, m, i, p_row, q_row):
        return p_row, 1.0

    monkeypatch.setattr(ots, "next_residual", no_reduction)
    fc, ns = _links({0: [1, 2]}, 3)
    law = _enumerate([P0, P1, P1], [Q0, Q0, Q0], fc, ns, {1: 0, 2: 0}, grid=12)
    first, _ = _marginal(law, 0)
    assert first != {0: Fraction(1, 2), 1: Fraction(3, 10), 2: Fraction(1, 5)}


def test_monte_carlo_bushy_tree():
    """V = 6, a root with three children, the first with two children and the
    second with one (7 nodes); random target and draft rows; 40000 rounds with
    drafts drawn from q.  The first token's law is p0 and the second token's,
    after an accepted first child, is that child's row (total variation below
    0.02; about 0.006 expected)."""
    rng = np.random.default_rng(7)
    V, N, R = 6, 7, 40000
    children = {0: [1, 2, 3], 1: [4, 5], 2: [6]}
    parent = {c: par for par, ks in children.items() for c in ks}
    fc, ns = _links(children, N)
    rows_p = rng.dirichlet(np.ones(V), size=N).astype(np.float32)
    rows_q = rng.dirichlet(np.ones(V), size=N).astype(np.float32)
    P = np.broadcast_to(rows_p, (R, N, V)).copy()
    Q = np.broadcast_to(rows_q, (R, N, V)).copy()
    d = np.zeros((R, N), np.int32)
    for c in range(1, N):
        w = rows_q[parent[c]].astype(np.float64)
        d[:, c] = rng.choice(V, size=R, p=w / w.sum())
    u = rng.random((R, N)).astype(np.float32)
    r = oracle.tree_sample_verify(P, Q, d, np.broadcast_to(fc, (R, N)), np.broadcast_to(ns, (R, N)), u)
    first = np.bincount(r["out_tokens"][:, 0], minlength=V) / R
    assert 0.5 * np.abs(first - rows_p[0] / rows_p[0].sum()).sum() < 0.02
    # second token after the first child was accepted (path 0 -> 1)
    sel = r["path"][:, 1] == 1
    assert sel.sum() > 2000
    second = np.bincount(r["out_tokens"][sel, 1], minlength=V) / sel.sum()
    assert 0.5 * np.abs(second - rows_p[1] / rows_p[1].sum()).sum() < 0.03
    # kept slots: the root and the accepted nodes, one per emitted token
    for b in range(50):
        e = int(r["emit_count"][b])
        pth = r["path"][b, :e].tolist()
        assert pth[0] == 0 and all(parent[c] == a for a, c in zip(pth, pth[1:]))
        assert r["accept_len"][b] == e - 1


def test_links_budget_eos_and_degenerate_rows():
    fc, ns = _links({0: [1, 2]}, 3)
    p = _rows([P0, P1, P1])[None]
    q = _rows([Q0, Q0, Q0])[None]
    d = np.array([[0, 0, 1]], np.int32)
    u = np.array([[0.5, 0.1, 0.1]], np.float32)                 # child 1 accepted
    r = oracle.tree_sample_verify(p, q, d, fc, ns, u)
    assert r["out_tokens"][0, :2].tolist()[0] == 0 and r["emit_count"][0] == 2
    r = oracle.tree_sample_verify(p, q, d, fc, ns, u, eos_id=0)  # EOS accepted: stop, no draw
    assert r["emit_count"][0] == 1 and r["final_mass"][0] == 0.0 and r["path"][0, 0] == 0
    r = oracle.tree_sample_verify(p, q, d, fc, ns, u, remaining=np.array([1], np.int32))
    assert r["emit_count"][0] == 1
    r = oracle.tree_sample_verify(p, q, d, fc, ns, u, remaining=np.array([0], np.int32))
    assert r["emit_count"][0] == 0 and r["status"][0] == 0
    bad = ns.copy()
    bad[0, 2] = 1                                                 # a backward link
    r = oracle.tree_sample_verify(p, q, d, fc, bad, u)
    assert r["emit_count"][0] == 0 and r["status"][0] == oracle.ST_BAD_STATE
    d2 = np.array([[0, 7, 1]], np.int32)                          # child 1 out of range: rejected
    r = oracle.tree_sample_verify(p, q, d2, fc, ns, np.array([[0.5, 0.0, 0.99]], np.float32))
    assert r["status"][0] & oracle.ST_DRAFT_OOR
    # p == q at the root and both children rejected (out of range): each
    # rejection leaves no residual, so the residual stays p and the draw is
    # from p itself
    r = oracle.tree_sample_verify(q.copy(), q, np.array([[0, 9, 9]], np.int32), fc, ns,
                                  np.array([[0.05, 0.0, 0.0]], np.float32))
    assert r["status"][0] == oracle.ST_RESID_ZERO | oracle.ST_DRAFT_OOR
    assert r["emit_count"][0] == 1 and r["accept_len"][0] == 0
    assert r["out_tokens"][0, 0] == 0                             # u = 0.05 of q0 = (0.2, 0.2, 0.6)
