"""Pins for the tree-verification oracle: the linear chain reduces to the
pinned greedy oracle; a hand-worked tree; the path properties on random trees;
and the compacted KV equals per-sequence decoding after the commit."""
import numpy as np
import pytest

import oracle
from oracle.tree import chain_links, compact_tree_slots, tree_verify
from workloads import fill_kv_np, kv_bits_np, planted_greedy


def _random_tree(rng, N, V, branching=3):
    """Topologically ordered random tree: node i's parent is below i."""
    parent = [-1] + [int(rng.integers(max(0, i - branching), i)) for i in range(1, N)]
    fc = np.full(N, -1, np.int32)
    ns = np.full(N, -1, np.int32)
    last = {}
    for i in range(1, N):
        p = parent[i]
        if fc[p] == -1:
            fc[p] = i
        else:
            ns[last[p]] = i
        last[p] = i
    draft = np.concatenate([[0], rng.integers(0, V, N - 1)]).astype(np.int32)
    return parent, fc, ns, draft


@pytest.mark.parametrize("eos,budget", [(-1, False), (7, False), (-1, True)])
def test_linear_chain_is_greedy_verification(eos, budget):
    rng = np.random.default_rng(1)
    B, k, V = 40, 5, 30
    g = planted_greedy(rng, rng, B, k, V, 1.0, "f32", rng.uniform(0.3, 1.0, B))
    rem = rng.integers(0, k + 3, B) if budget else None
    fc, ns = chain_links(B, k + 1)
    draft = np.concatenate([np.zeros((B, 1), np.int32), g["drafts"]], axis=1)
    t = tree_verify(g["logits"], "f32", draft, fc, ns, eos_id=eos, remaining=rem)
    ref = oracle.greedy_verify(g["logits"], "f32", g["drafts"], eos_id=eos, remaining=rem)
    for key in ["accept_len", "emit_count", "emit_offsets", "status"]:
        assert np.array_equal(t[key], ref[key]), key
    assert np.array_equal(t["out_tokens"], ref["out_tokens"])
    for b in range(B):
        e = int(t["emit_count"][b])
        assert t["path"][b, :e].tolist() == list(range(e))


def test_worked_tree():
    # root -> A(5), B(7), E(7); A -> C(9); B -> D(3)    (node ids: A1 B2 C3 D4 E5)
    V = 12
    fc = np.array([[1, 3, 4, -1, -1, -1]])
    ns = np.array([[-1, 2, 5, -1, -1, -1]])
    draft = np.array([[0, 5, 7, 9, 3, 7]])
    x = np.full((1, 6, V), -1.0, np.float32)
    x[0, 0, 7] = 2.0            # root: 7 -> B (the first child proposing 7; E also proposes it)
    x[0, 2, 3] = 1.0            # B: 3 -> D
    x[0, 4, 11] = 0.5           # D (leaf): bonus 11
    t = tree_verify(x, "f32", draft, fc, ns)
    assert t["out_tokens"][0, :3].tolist() == [7, 3, 11]
    assert t["emit_count"][0] == 3 and t["accept_len"][0] == 2
    assert t["path"][0, :3].tolist() == [0, 2, 4]
    x[0, 2, 3] = -5.0
    x[0, 2, 8] = 1.0            # B: 8, no child proposes it -> correction
    t = tree_verify(x, "f32", draft, fc, ns)
    assert t["out_tokens"][0, :2].tolist() == [7, 8] and t["accept_len"][0] == 1
    assert t["path"][0, :2].tolist() == [0, 2]


def test_random_tree_path_properties():
    rng = np.random.default_rng(2)
    for _ in range(300):
        N, V = int(rng.integers(1, 12)), int(rng.integers(2, 6))
        parent, fc, ns, draft = _random_tree(rng, N, V)
        x = rng.standard_normal((1, N, V)).astype(np.float32)
        t = tree_verify(x, "f32", draft[None], fc[None], ns[None])
        e, a = int(t["emit_count"][0]), int(t["accept_len"][0])
        path = t["path"][0, :e].tolist()
        out = t["out_tokens"][0, :e].tolist()
        assert path[0] == 0 and e == a + 1 and len(path) == e
        for j in range(e):
            assert out[j] == int(np.argmax(x[0, path[j]]))
        for j in range(1, e):
            assert parent[path[j]] == path[j - 1] and draft[path[j]] == out[j - 1]
        last = path[-1]
        kids = [i for i in range(N) if parent[i] == last]
        assert all(draft[c] != out[-1] for c in kids)          # stopped: nothing matches


def test_bad_links_report_status():
    fc = np.array([[2, -1, 1]])                              # link backwards (2 -> 1)
    ns = np.full((1, 3), -1)
    t = tree_verify(np.zeros((1, 3, 4), np.float32), "f32", np.array([[0, 1, 2]]), fc, ns)
    assert t["status"][0] & oracle.ST_BAD_STATE and t["emit_count"][0] == 0


def test_compacted_tree_commit_matches_per_sequence_decoding():
    rng = np.random.default_rng(3)
    B, N, V, L, H, D = 6, 9, 6, 2, 2, 8
    P = rng.integers(2, 15, B)
    toks = [rng.integers(0, V, int(p)).tolist() for p in P]
    model = oracle.UnbatchedModel(toks)
    n = model.n_all()
    E = int(n.max())
    C = E + N + 2
    grid = np.zeros((B, int(P.max())), np.int64)
    for b in range(B):
        grid[b, :len(toks[b])] = toks[b]
    kv = fill_kv_np(L, H, D, B, C, E, n, grid, "bf16")
    trees = [_random_tree(rng, N, V) for _ in range(B)]
    fc = np.stack([t[1] for t in trees])
    ns = np.stack([t[2] for t in trees])
    draft = np.stack([t[3] for t in trees])
    # the tree forward: node i's KV (its token at position n_b + depth(i)) in slot E + i
    for b in range(B):
        parent = trees[b][0]
        for i in range(N):
            depth, j = 0, i
            while parent[j] != -1:
                j, depth = parent[j], depth + 1
            tok = model.tokens[b][-1] if i == 0 else int(draft[b, i])
            pos = int(n[b]) + depth
            plane = np.arange(L * 2 * H).reshape(L, 2, H)
            kv[:, :, b, :, E + i, :] = kv_bits_np(b, pos, tok, plane[..., None], np.arange(D), "bf16")
    x = rng.standard_normal((B, N, V)).astype(np.float32)
    for b in range(B):                                        # bias toward acceptance
        for i in range(N):
            kids = [c for c in range(N) if trees[b][0][c] == i]
            if kids and rng.random() < 0.8:
                x[b, i, draft[b, kids[-1]]] += 5.0
    t = tree_verify(x, "f32", draft, fc, ns)
    kv2 = compact_tree_slots(kv, E, t["path"], t["emit_count"])
    com = oracle.commit_realign(kv2, E, n, t["emit_count"], N - 1)
    model.commit(t["out_tokens"], t["emit_count"])
    content = lambda b, pos, tok, plane, d: kv_bits_np(b, pos, tok, plane, d, "bf16")
    assert model.check(com["kv"], com["pos"], com["mask"], com["E_new"], content) == []
    assert t["accept_len"].max() >= 2                         # some sequences went deep
    # negative control: committing the first e slots without compaction
    wrong = oracle.commit_realign(kv, E, n, t["emit_count"], N - 1)
    moved = any(t["path"][b, :int(t["emit_count"][b])].tolist() != list(range(int(t["emit_count"][b])))
                for b in range(B))
    assert moved and model.check(wrong["kv"], wrong["pos"], wrong["mask"], wrong["E_new"], content)
