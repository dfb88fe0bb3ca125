"""GPU parity of greedy tree verification (spec_verify_tree) and of the
compaction of the accepted path's KV slots (spec_compact_tree_kv) against the
oracle: tokens, counts, paths, offsets and status must be identical, and the
compacted cache bit-identical; a linear chain must equal spec_verify_greedy;
a tree round followed by the realigning commit must leave the cache in the
state per-sequence decoding implies."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.tree import chain_links
from tests._gpu import (DEV, commit, compact_tree, host, i32, kv_bits, logits_to_device, note, requires_gpu,
                        verify_greedy, verify_tree)

pytestmark = [pytest.mark.gpu, requires_gpu]

KEYS = ["accept_len", "emit_count", "out_tokens", "path", "emit_offsets", "status"]


def _tree_case(seed, B, N, V, dt, alpha=0.8, branching=3, sd=2.0):
    rng = np.random.default_rng(seed)
    return W.planted_tree(rng, rng, B, N, V, sd, dt, alpha, branching)


def _check_tree(g, eos=-1, rem=None, ws_key=None):
    ref = oracle.tree_verify(g["logits"], g["dtype"], g["draft"], g["first_child"], g["next_sibling"],
                             eos_id=eos, remaining=rem)
    got = host(verify_tree(logits_to_device(g["logits"], g["dtype"]), g["draft"], g["first_child"],
                           g["next_sibling"], eos_id=eos, remaining=rem, ws_key=ws_key))
    for key in KEYS:
        assert np.array_equal(got[key], ref[key]), key
    return ref


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,N,V", [(1, 1, 7), (3, 2, 100), (16, 9, 1000), (5, 16, 4099), (37, 64, 300),
                                   (4, 256, 64), (300, 5, 50), (2, 16, 128256)])
def test_tree_verify_matches_oracle(B, N, V, dt):
    note(f"tree verify B={B} N={N} V={V} {dt}")
    ref = _check_tree(_tree_case(B * 1000 + N, B, N, V, dt))
    if N >= 9 and B >= 5:
        assert ref["accept_len"].max() >= 2                 # some paths go deep


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_tree_verify_eos_budget_and_ties(dt):
    rng = np.random.default_rng(5)
    for it in range(12):
        B, N, V = int(rng.integers(1, 40)), int(rng.integers(1, 30)), int(rng.integers(2, 40))
        g = _tree_case(100 + it, B, N, V, dt, alpha=0.9, branching=int(rng.integers(1, 5)), sd=0.5)
        eos = int(rng.integers(0, V)) if it % 3 else -1
        rem = rng.integers(0, N + 2, B) if it % 2 else None
        note(f"tree eos/budget {it}: B={B} N={N} V={V} eos={eos} {dt}")
        _check_tree(g, eos, rem)


def test_tree_verify_many_sequences_cross_tiles():
    """More sequences than one pass of the commit kernel holds (1024 rows)."""
    g = _tree_case(7, 700, 12, 33, "bf16", alpha=0.9)
    note("tree verify B=700 N=12")
    _check_tree(g, rem=np.random.default_rng(7).integers(0, 14, 700))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_linear_chain_equals_greedy_verification(dt):
    rng = np.random.default_rng(8)
    B, k, V = 24, 7, 32000
    g = W.planted_greedy(rng, rng, B, k, V, 2.0, dt, rng.uniform(0.3, 1.0, B))
    rem = rng.integers(0, k + 3, B)
    fc, ns = chain_links(B, k + 1)
    draft = np.concatenate([np.zeros((B, 1), np.int32), g["drafts"]], axis=1)
    x = logits_to_device(g["logits"], dt)
    note(f"tree chain vs greedy B={B} k={k} {dt}")
    t = host(verify_tree(x, draft, fc, ns, eos_id=3, remaining=rem))
    r = host(verify_greedy(x, g["drafts"], eos_id=3, remaining=rem))
    for key in ["accept_len", "emit_count", "out_tokens", "emit_offsets", "status"]:
        assert np.array_equal(t[key], r[key]), key
    for b in range(B):
        e = int(t["emit_count"][b])
        assert t["path"][b, :e].tolist() == list(range(e))


def test_tree_verify_bad_links_and_draft_ids():
    g = _tree_case(9, 6, 8, 50, "f32", alpha=1.0)
    fc, ns, draft = g["first_child"].copy(), g["next_sibling"].copy(), g["draft"].copy()
    fc[1, 3] = 2                    # backwards
    ns[2, 7] = 8                    # past the tree
    fc[3, 0] = 0                    # self loop
    draft[4, 5] = 50                # out of range: never matches, flagged
    draft[5, 2] = -3
    g2 = dict(g, first_child=fc, next_sibling=ns, draft=draft)
    note("tree verify bad links")
    ref = _check_tree(g2)
    assert (ref["status"][1:4] & oracle.ST_BAD_STATE).all() and (ref["emit_count"][1:4] == 0).all()
    assert ref["status"][4] == oracle.ST_DRAFT_OOR and ref["status"][5] == oracle.ST_DRAFT_OOR


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _random_kv(rng, shape, dt):
    bits = rng.integers(0, 1 << 16 if dt == "bf16" else 1 << 31, shape)
    a = bits.astype(np.int16 if dt == "bf16" else np.int32)
    return torch.from_numpy(a).to(DEV).view(_tdt(dt))


def test_compaction_matches_oracle():
    rng = np.random.default_rng(11)
    for it in range(40):
        dt = "bf16" if it % 2 else "f32"
        L, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        D = int(rng.choice([1, 3, 8, 64, 128]))
        B, N = int(rng.integers(1, 9)), int(rng.integers(1, 40))
        E = int(rng.integers(0, 20))
        C = E + N + int(rng.integers(0, 4))
        paths = np.full((B, N), -1, np.int32)
        e = rng.integers(0, N + 1, B).astype(np.int32)
        for b in range(B):
            if e[b]:
                rest = np.sort(rng.choice(np.arange(1, N), int(e[b]) - 1, replace=False)) if N > 1 else []
                paths[b, :e[b]] = np.concatenate([[0], rest])
        kv = _random_kv(rng, (L, 2, B, H, C, D), dt)
        pre = kv_bits(kv)
        note(f"compact {it}: L={L} H={H} D={D} B={B} N={N} E={E} C={C} {dt}")
        st = host(dict(s=compact_tree(kv, N, E, paths, e)))["s"]
        assert (st == 0).all()
        assert np.array_equal(kv_bits(kv), oracle.compact_tree_slots(pre, E, paths, e))


@pytest.mark.parametrize("L,B,H,D,N,dt", [(8, 2, 101, 8, 7, "f32"),      # heads split across workgroups, ragged
                                           (1, 3, 3, 128, 256, "bf16"),   # longest paths: many passes
                                           (2, 1, 1, 5, 33, "bf16")])     # 10-byte columns
def test_compaction_shapes(L, B, H, D, N, dt):
    rng = np.random.default_rng(L * 100 + N)
    E = 3
    C = E + N + 1
    e = np.array([N, N // 2, 1][:B], np.int32)
    paths = np.full((B, N), -1, np.int32)
    for b in range(B):
        rest = np.sort(rng.choice(np.arange(1, N), int(e[b]) - 1, replace=False)) if e[b] > 1 else []
        paths[b, :e[b]] = np.concatenate([[0], rest])
    if B > 1:
        paths[1, :e[1]] = np.concatenate([[0], np.arange(N - int(e[1]) + 1, N)])    # skips to the far end
    kv = _random_kv(rng, (L, 2, B, H, C, D), dt)
    pre = kv_bits(kv)
    note(f"compact shape L={L} B={B} H={H} D={D} N={N} {dt}")
    st = host(dict(s=compact_tree(kv, N, E, paths, e)))["s"]
    assert (st == 0).all()
    assert np.array_equal(kv_bits(kv), oracle.compact_tree_slots(pre, E, paths, e))


def test_compaction_rejects_bad_sequences_and_leaves_them():
    rng = np.random.default_rng(12)
    L, H, D, B, N, E = 1, 2, 64, 5, 6, 4
    C = E + N
    paths = np.array([[0, 2, 3, -1, -1, -1],       # fine
                      [1, 2, -1, -1, -1, -1],      # does not start at the root
                      [0, 3, 3, -1, -1, -1],       # not increasing
                      [0, 1, 2, 3, 4, 5],          # e = 7 > N
                      [0, 6, -1, -1, -1, -1]],     # node past the tree
                     np.int32)
    e = np.array([3, 2, 3, 7, 2], np.int32)
    kv = _random_kv(rng, (L, 2, B, H, C, D), "bf16")
    pre = kv_bits(kv)
    note("compact bad sequences")
    st = host(dict(s=compact_tree(kv, N, E, paths, e)))["s"]
    assert st.tolist() == [0] + [oracle.ST_BAD_STATE] * 4
    want = pre.copy()
    want[:, :, :1] = oracle.compact_tree_slots(pre[:, :, :1], E, paths[:1], e[:1])
    assert np.array_equal(kv_bits(kv), want)
    # end column too far right for N slots: every sequence is left alone
    kv2 = _random_kv(rng, (L, 2, B, H, C, D), "f32")
    pre2 = kv_bits(kv2)
    st = host(dict(s=compact_tree(kv2, N, E + 1, paths, e)))["s"]
    assert (st == oracle.ST_BAD_STATE).all() and np.array_equal(kv_bits(kv2), pre2)


def _depths(parent):
    d = np.zeros(len(parent), np.int64)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_tree_round_then_commit_matches_per_sequence_decoding(dt):
    """Tree verify, compaction and the realigning commit, all on the GPU: the
    cache, positions and mask must be those of decoding each sequence alone."""
    rng = np.random.default_rng(13)
    B, N, V, L, H, D = 9, 12, 40, 2, 2, 64
    P = rng.integers(2, 30, B)
    toks = [rng.integers(0, V, int(p)).tolist() for p in P]
    model = oracle.UnbatchedModel(toks)
    n = model.n_all()
    E = int(n.max())
    C = E + N + 3
    grid = np.zeros((B, int(P.max())), np.int64)
    for b in range(B):
        grid[b, :len(toks[b])] = toks[b]
    kv_np = W.fill_kv_np(L, H, D, B, C, E, n, grid, dt)
    g = _tree_case(14, B, N, V, "f32", alpha=0.85)
    plane = np.arange(L * 2 * H).reshape(L, 2, H)
    for b in range(B):                               # the tree forward's slots
        depth = _depths(g["parent"][b])
        for i in range(N):
            tok = model.tokens[b][-1] if i == 0 else int(g["draft"][b, i])
            kv_np[:, :, b, :, E + i, :] = W.kv_bits_np(b, int(n[b]) + int(depth[i]), tok, plane[..., None],
                                                       np.arange(D), dt)
    view = np.int16 if dt == "bf16" else np.int32
    kv = torch.from_numpy(kv_np.view(view)).to(DEV).view(_tdt(dt))
    note(f"tree round + commit {dt}")
    t = verify_tree(logits_to_device(g["logits"], "f32"), g["draft"], g["first_child"], g["next_sibling"])
    st = compact_tree(kv, N, E, t["path"], t["emit_count"])
    c = host(commit(kv, N - 1, E, n, t["emit_count"]))
    th = host(t)
    assert (host(dict(s=st))["s"] == 0).all() and (c["status"] == 0).all()
    assert th["accept_len"].max() >= 2
    model.commit(th["out_tokens"], th["emit_count"])
    content = lambda b, pos, tok, pl, d: W.kv_bits_np(b, pos, tok, pl, d, dt)
    assert model.check(kv_bits(kv), c["pos"], c["mask"], int(c["end_col"][0]), content) == []


def test_tree_bench_shape():
    """The benchmark's tree shape: B=32 sequences of 16-node trees over V=128256
    bf16 logits (generated as the benchmark does), verified exactly; then the
    compaction in the full 32 x 8 x 128 bf16 cache, checked on sampled planes."""
    cfg = W.workload(3)
    g3 = W.kv_geometry(3)
    B, NT, V = g3["B"], 16, cfg["V"]
    g = W.planted_tree(W.stream(3, "logits", 0, 1), W.stream(3, "drafts", 0, 1), B, NT, V, cfg["logit_sd"],
                       "bf16", W.alphas(3), 3)
    note(f"tree bench shape verify B={B} N={NT} V={V}")
    ref = _check_tree(g)
    assert ref["accept_len"].max() >= 2
    L, H, D, E = g3["L"], g3["H"], g3["D"], g3["E"]
    C = E + NT
    note(f"tree bench shape compaction L={L} H={H} D={D} C={C}")
    kv = torch.empty((L, 2, B, H, C, D), dtype=torch.bfloat16, device=DEV)
    iv = kv.view(torch.int16)
    gen = torch.Generator(device=DEV).manual_seed(5)
    iv[:, :, :, :, E:, :] = torch.randint(-32768, 32767, (L, 2, B, H, NT, D), dtype=torch.int16, device=DEV,
                                          generator=gen)
    rng = np.random.default_rng(6)
    planes = [(int(rng.integers(L)), int(rng.integers(2)), int(rng.integers(B)), int(rng.integers(H)))
              for _ in range(48)]
    before = [iv[l, c, b, h, E:, :].cpu().numpy() for l, c, b, h in planes]
    st = host(dict(s=compact_tree(kv, NT, E, ref["path"], ref["emit_count"])))["s"]
    assert (st == 0).all()
    for (l, c, b, h), pre in zip(planes, before):
        got = iv[l, c, b, h, E:, :].cpu().numpy()
        # the oracle's compaction of this one plane (its columns E.. as a
        # cache of one layer, one K/V half, one sequence and one head)
        want = oracle.compact_tree_slots(pre[None, None, None, None], 0, ref["path"][b:b + 1],
                                         ref["emit_count"][b:b + 1])[0, 0, 0, 0]
        assert np.array_equal(got, want), (l, c, b, h)
    del kv, iv
    torch.cuda.empty_cache()


def test_tree_incomplete_when_the_wait_bound_is_reached():
    """A one-poll wait bound makes the tree commit stop waiting before the
    chunk results of its first tile have arrived: the call still ends, the
    sequences it gave up on carry SPEC_ST_INCOMPLETE, and every sequence whose
    status does not carry it is exact.  With the default bound restored, the
    same workspace (zero-filled again) gives exact results."""
    import speculative_decoding_verification_04_amd as sv
    from tests._gpu import ws
    B, N, V = 64, 16, 128256
    note(f"tree wait bound of one poll B={B} N={N} V={V}")
    g = _tree_case(91, B, N, V, "bf16")
    ref = oracle.tree_verify(g["logits"], "bf16", g["draft"], g["first_child"], g["next_sibling"])
    x = logits_to_device(g["logits"], "bf16")
    w = ws(sv.spec_verify_tree_workspace_bytes(B, N, V, sv.SPEC_BF16), ("greedy", "tree_bound"))
    prev = sv.spec_set_wait_bound(1)
    try:
        out = host(verify_tree(x, g["draft"], g["first_child"], g["next_sibling"], ws_key="tree_bound"))
    finally:
        assert sv.spec_set_wait_bound(prev) == 1
    torch.cuda.synchronize()
    w.zero_()                       # late chunk results may have landed after the commit gave up
    inc = (out["status"] & sv.SPEC_ST_INCOMPLETE) != 0
    assert inc.any()
    for key in ("accept_len", "emit_count", "out_tokens", "path"):
        assert np.array_equal(out[key][~inc], ref[key][~inc]), key
    again = host(verify_tree(x, g["draft"], g["first_child"], g["next_sibling"], ws_key="tree_bound"))
    for key in KEYS:
        assert np.array_equal(again[key], ref[key]), key
