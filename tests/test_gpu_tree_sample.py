"""GPU parity of spec_verify_tree_sample against the oracle
(oracle.tree_sample_verify): accept lengths, emitted tokens, kept paths,
offsets and status bit-exact, the drawn vector's mass within float64
rounding of the oracle's correctly rounded sum; random trees (drafts drawn
from the parent's q) from tiny to full-vocabulary rows, many siblings (many
residual levels at one node), ragged and unaligned rows, EOS, budgets,
invalid links, out-of-range drafts, q(x) = 0 and rows without residual
mass; and a chain tree against spec_verify_sample, bit for bit.  Every case
runs twice: one workgroup per sequence (no workspace), and, where the shape
allows it, several workgroups per sequence exchanging chunk masses through
the workspace, which every call must leave zero-filled."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_04_amd as sv
import workloads as W
from oracle.tree import chain_links
from tests._gpu import DEV, host, i32, note, requires_gpu, verify_sample, ws

pytestmark = [pytest.mark.gpu, requires_gpu]

KEYS = ["accept_len", "emit_count", "out_tokens", "path", "emit_offsets", "status"]


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def run(g, eos_id=-1, remaining=None, p_dev=None, q_dev=None, coop=False):
    B, N, V = g["p"].shape
    w = None
    if coop:
        nb = sv.spec_verify_tree_sample_workspace_bytes(B, N, V)
        w = ws(nb, ("tree_sample", None)) if nb else None
    out = dict(accept_len=torch.full((B,), -7, dtype=torch.int32, device=DEV),
               emit_count=torch.full((B,), -7, dtype=torch.int32, device=DEV),
               out_tokens=torch.full((B, N), -7, dtype=torch.int32, device=DEV),
               path=torch.full((B, N), -7, dtype=torch.int32, device=DEV),
               emit_offsets=torch.full((B + 1,), -7, dtype=torch.int32, device=DEV),
               final_mass=torch.full((B,), -7.0, dtype=torch.float64, device=DEV),
               status=torch.full((B,), -7, dtype=torch.int32, device=DEV))
    sv.spec_verify_tree_sample(
        _dev_f32(g["p"]) if p_dev is None else p_dev, _dev_f32(g["q"]) if q_dev is None else q_dev,
        i32(g["draft"]), i32(g["first_child"]), i32(g["next_sibling"]), _dev_f32(g["uniforms"]),
        out["accept_len"], out["emit_count"], out["out_tokens"], out["path"], eos_id=eos_id,
        remaining=None if remaining is None else i32(remaining), emit_offsets=out["emit_offsets"],
        final_mass=out["final_mass"], status=out["status"], ws=w)
    got = host(out)
    if w is not None:
        assert int(torch.count_nonzero(w).item()) == 0          # slots and flags clear again
    return got


def compare(g, eos_id=-1, remaining=None, **kw):
    """Both launch shapes against the oracle; they must also agree with each
    other bit for bit (the same sums in the same order)."""
    ref = oracle.tree_sample_verify(g["p"], g["q"], g["draft"], g["first_child"], g["next_sibling"],
                                    g["uniforms"], eos_id=eos_id, remaining=remaining)
    gots = [run(g, eos_id, remaining, coop=c, **kw) for c in (False, True)]
    for got in gots:
        for k in KEYS:
            assert np.array_equal(got[k], ref[k]), (k, got[k], ref[k])
        fm, rm = got["final_mass"], ref["final_mass"]
        fin = np.isfinite(rm)
        assert np.array_equal(np.isfinite(fm), fin)
        assert np.allclose(fm[fin], rm[fin], rtol=1e-12, atol=0)
    for k in gots[0]:
        assert np.array_equal(gots[0][k], gots[1][k], equal_nan=True), k
    return gots[1], ref


@pytest.mark.parametrize("B,N,V,branching", [
    (4, 8, 1000, 3), (8, 16, 151936, 3), (3, 32, 4099, 5), (5, 64, 37, 8), (2, 256, 300, 2), (6, 5, 8192, 4),
    (100, 6, 9000, 3),
])
def test_random_trees(B, N, V, branching):
    rng = np.random.default_rng(1000 * N + B)
    for r in range(3):
        note(f"tree sample B={B} N={N} V={V} branching={branching} round {r}")
        g = W.sampled_tree(rng, B, N, V, branching=branching)
        got, _ = compare(g)
        assert (got["emit_count"] >= 1).all()


def test_many_siblings():
    """A root with 40 children and draft rows far from the target: most tries
    are rejected, so the residual goes through many levels at one node."""
    rng = np.random.default_rng(77)
    B, N, V = 6, 41, 2000
    note(f"tree sample many siblings B={B} N={N} V={V}")
    g = W.sampled_tree(rng, B, N, V, eps_sd=4.0, branching=N)   # every node's parent: the root
    g["first_child"][:] = -1
    g["next_sibling"][:] = -1
    g["first_child"][:, 0] = 1
    g["next_sibling"][:, 1:N - 1] = np.arange(2, N)
    qrows = g["q"][:, 0].astype(np.float64)
    ud = rng.random((B, N))
    for b in range(B):
        c = np.cumsum(qrows[b])
        g["draft"][b, 1:] = np.minimum(np.searchsorted(c, ud[b, 1:] * c[-1], side="right"), V - 1)
    got, ref = compare(g)
    assert (ref["accept_len"] <= 1).all()
    assert (got["path"][:, 0] == 0).all()


def test_chain_is_spec_verify_sample():
    """A chain tree over the stochastic workload's inputs gives what
    spec_verify_sample gives on the linear layout, bit for bit (final mass
    included)."""
    note("tree sample chain vs spec_verify_sample")
    r = W.sample_round(2, round_=3)
    p, q, d, u = r["p"], r["q"], r["drafts"], r["uniforms"]
    B, kp1, V = p.shape
    k = kp1 - 1
    fc, ns = chain_links(B, kp1)
    g = dict(p=p, q=np.concatenate([q, np.zeros((B, 1, V), np.float32)], axis=1),
             draft=np.concatenate([np.zeros((B, 1), np.int32), d], axis=1), first_child=fc, next_sibling=ns,
             uniforms=np.concatenate([u[:, k:], u[:, :k]], axis=1))
    got, _ = compare(g)
    lin = host(verify_sample(_dev_f32(p), _dev_f32(q), d, u))
    for key in ["accept_len", "emit_count", "emit_offsets", "status"]:
        assert np.array_equal(got[key], lin[key]), key
    assert np.array_equal(got["out_tokens"], lin["out_tokens"])
    assert np.array_equal(got["final_mass"], lin["final_mass"])


def test_chain_is_spec_verify_sample_on_long_rows():
    """Rows of more than 256 chunks (V = 1200003: 293 chunks of 4096), where
    the chunk masses are added in runs of two per lane: still bit for bit."""
    note("tree sample chain vs spec_verify_sample, V=1200003")
    r = W.sample_round(2, round_=1, B=2, V=1200003, k=2)
    p, q, d, u = r["p"], r["q"], r["drafts"], r["uniforms"]
    B, kp1, V = p.shape
    k = kp1 - 1
    fc, ns = chain_links(B, kp1)
    g = dict(p=p, q=np.concatenate([q, np.zeros((B, 1, V), np.float32)], axis=1),
             draft=np.concatenate([np.zeros((B, 1), np.int32), d], axis=1), first_child=fc, next_sibling=ns,
             uniforms=np.concatenate([u[:, k:], u[:, :k]], axis=1))
    got, _ = compare(g)
    lin = host(verify_sample(_dev_f32(p), _dev_f32(q), d, u))
    for key in ["accept_len", "emit_count", "emit_offsets", "status", "out_tokens", "final_mass"]:
        assert np.array_equal(got[key], lin[key]), key


def test_edge_cases():
    rng = np.random.default_rng(5)
    B, N, V = 6, 6, 513
    note("tree sample edge cases")
    g = W.sampled_tree(rng, B, N, V)
    # EOS at an accepted draft, budgets (0, 1, none), a lone root
    for eos in (-1, int(g["draft"][0, 1])):
        for rem in (None, np.array([0, 1, 2, -1, 3, 1], np.int32)):
            compare(g, eos_id=eos, remaining=rem)
    g1 = {k: (v[:, :1] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in g.items()}
    g1["first_child"] = np.full((B, 1), -1, np.int32)
    g1["next_sibling"] = np.full((B, 1), -1, np.int32)
    got, _ = compare(g1)                                    # N = 1: the bonus from the root row
    assert (got["emit_count"] == 1).all() and (got["accept_len"] == 0).all()
    # invalid links, out-of-range drafts, q(x) = 0 at a drafted token, p == q
    h = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in g.items()}
    h["next_sibling"][0, 3] = 2                              # backward link: that sequence emits nothing
    h["draft"][1, 1:] = V + 4
    c = int(h["first_child"][2, 0])
    h["q"][2, 0, h["draft"][2, c]] = 0.0
    h["p"][3] = h["q"][3]                                    # no residual mass anywhere
    got, ref = compare(h)
    assert ref["status"][0] == oracle.ST_BAD_STATE and got["emit_count"][0] == 0
    assert ref["status"][1] & oracle.ST_DRAFT_OOR
    assert ref["status"][2] & oracle.ST_Q_ZERO


def test_unaligned_rows_and_repeatable():
    """Rows that start off a 16-byte boundary take the scalar loads; 20 calls
    give identical outputs."""
    rng = np.random.default_rng(9)
    B, N, V = 3, 9, 1001
    note("tree sample unaligned + repeat")
    g = W.sampled_tree(rng, B, N, V)
    pf = torch.empty(B * N * V + 1, dtype=torch.float32, device=DEV)
    qf = torch.empty(B * N * V + 1, dtype=torch.float32, device=DEV)
    pf[1:] = _dev_f32(g["p"]).reshape(-1)
    qf[1:] = _dev_f32(g["q"]).reshape(-1)
    pd, qd = pf[1:].view(B, N, V), qf[1:].view(B, N, V)
    first, _ = compare(g, p_dev=pd, q_dev=qd)
    for it in range(19):
        again = run(g, p_dev=pd, q_dev=qd)
        for k in first:
            assert np.array_equal(first[k], again[k]), k
