"""The calls launch kernels only (no allocation, copy or fill), so a caller may
capture them in a HIP graph.  Each capture here is replayed several times, with
eager work and synchronisation between replays, and every replay must give the
eager call's outputs bit for bit."""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_04_amd as sv
import workloads as W
from tests._gpu import DEV, i32, logits_to_device, note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _replay_matches(fn, outs, replays=3, defined=None):
    """fn() writes into the tensors of `outs`; the graph of fn must reproduce
    them (only the part `defined(outs)` returns, per tensor, when given)."""
    fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for rep in range(replays):
        for o in outs:
            o.fill_(-7)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        views = defined(outs) if defined else outs
        wants = defined(want) if defined else want
        for o, w in zip(views, wants):
            assert torch.equal(o, w), rep


def test_greedy_and_tree_verify_replay():
    rng = np.random.default_rng(1)
    B, k, V = 8, 5, 32000
    gr = W.planted_greedy(rng, rng, B, k, V, 2.0, "bf16", 0.8)
    x = logits_to_device(gr["logits"], "bf16")
    d = i32(gr["drafts"])
    out = [torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B, k + 1, dtype=torch.int32, device=DEV), torch.empty(B + 1, dtype=torch.int32, device=DEV)]
    ws = sv.workspace(sv.spec_verify_greedy_workspace_bytes(B, k, V, sv.SPEC_BF16), DEV)
    note("graph: greedy verify")
    _replay_matches(lambda: sv.spec_verify_greedy(x, d, out[0], out[1], out[2], ws, emit_offsets=out[3]), out)
    g = W.planted_tree(rng, rng, B, 12, V, 2.0, "bf16", 0.8)
    z = logits_to_device(g["logits"], "bf16")
    dr, fc, ns = i32(g["draft"]), i32(g["first_child"]), i32(g["next_sibling"])
    tout = [torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
            torch.empty(B, 12, dtype=torch.int32, device=DEV), torch.empty(B, 12, dtype=torch.int32, device=DEV)]
    wst = sv.workspace(sv.spec_verify_tree_workspace_bytes(B, 12, V, sv.SPEC_BF16), DEV)
    note("graph: tree verify")
    _replay_matches(lambda: sv.spec_verify_tree(z, dr, fc, ns, tout[0], tout[1], tout[2], tout[3], wst), tout)


@pytest.mark.parametrize("K,P", [(50, 0.9), (0, 0.9), (0, 1.0)])
def test_stochastic_verify_replay(K, P):
    r = W.sample_round(2, B=4)
    B, k, V = r["B"], r["k"], r["V"]
    p, q = torch.from_numpy(r["p"]).to(DEV), torch.from_numpy(r["q"]).to(DEV)
    d, u = i32(r["drafts"]), torch.from_numpy(r["uniforms"]).to(DEV)
    out = [torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B, k + 1, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.float64, device=DEV),
           torch.empty(B + 1, dtype=torch.int32, device=DEV)]
    ws = sv.workspace(sv.spec_verify_sample_workspace_bytes(B, k, V), DEV)
    note("graph: stochastic verify")
    _replay_matches(lambda: sv.spec_verify_sample(p, q, d, u, out[0], out[1], out[2], ws, final_mass=out[3],
                                                  emit_offsets=out[4]), out)
    assert int(torch.count_nonzero(ws).item()) == 0          # the completion flags are clear again
    g = W.sample_logits(2, B=4)
    zt = torch.from_numpy(g["zt"]).to(DEV).to(torch.bfloat16)
    zd = torch.from_numpy(g["zd"]).to(DEV).to(torch.bfloat16)
    wsl = sv.workspace(sv.spec_verify_sample_logits_workspace_bytes(B, k, V), DEV)
    note(f"graph: stochastic verify from logits K={K} P={P}")
    _replay_matches(lambda: sv.spec_verify_sample_logits(zt, zd, d, u, out[0], out[1], out[2], wsl,
                                                         temperature=0.7, top_k=K, top_p=P, final_mass=out[3],
                                                         emit_offsets=out[4]),
                    out)


def test_tree_sample_replay():
    rng = np.random.default_rng(12)
    g = W.sampled_tree(rng, 6, 10, 5000)
    B, N = 6, 10
    p, q = torch.from_numpy(g["p"]).to(DEV), torch.from_numpy(g["q"]).to(DEV)
    d, fc, ns = i32(g["draft"]), i32(g["first_child"]), i32(g["next_sibling"])
    u = torch.from_numpy(g["uniforms"]).to(DEV)
    out = [torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B, N, dtype=torch.int32, device=DEV), torch.empty(B, N, dtype=torch.int32, device=DEV),
           torch.empty(B + 1, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.float64, device=DEV)]
    wst = sv.workspace(sv.spec_verify_tree_sample_workspace_bytes(B, N, 5000), DEV)
    note("graph: stochastic tree verify")
    _replay_matches(lambda: sv.spec_verify_tree_sample(p, q, d, fc, ns, u, out[0], out[1], out[2], out[3], wst,
                                                       emit_offsets=out[4], final_mass=out[5]), out)
    assert int(torch.count_nonzero(wst).item()) == 0


def test_paged_and_grouping_replay():
    g3 = W.kv_geometry(3)
    B, k, page = g3["B"], g3["k"], 16
    n = i32(g3["n"])
    e = i32(W.accept_counts(3, 0))
    maxp = (int(g3["n"].max()) + k + 1 + page - 1) // page
    bt = torch.arange(B * maxp, dtype=torch.int32, device=DEV).view(B, maxp)
    per = (k + page) // page
    out = [torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B * per, dtype=torch.int32, device=DEV), torch.empty(B + 1, dtype=torch.int32, device=DEV)]
    note("graph: paged commit")
    # the released list is defined up to its total (the last offset)
    _replay_matches(lambda: sv.spec_commit_paged(k, page, n, e, bt, out[0], out[1], out[2], out[3]), out,
                    defined=lambda o: [o[0], o[1], o[2][:int(o[3][-1].item())], o[3]])
    P = W.pool_lengths()
    L = i32(P)
    N = P.size
    gout = [torch.empty(N, dtype=torch.int32, device=DEV), torch.empty(N + 1, dtype=torch.int32, device=DEV),
            torch.empty(N, dtype=torch.int32, device=DEV), torch.empty(1, dtype=torch.int32, device=DEV),
            torch.empty(1, dtype=torch.int32, device=DEV)]
    note("graph: grouping")
    # batch_start / batch_len are defined up to the batch count
    _replay_matches(lambda: sv.spec_group_same_length(L, 8, 2, *gout), gout,
                    defined=lambda o: [o[0], o[1][:int(o[3].item()) + 1], o[2][:int(o[3].item())], o[3], o[4]])


def test_commit_and_compaction_replay():
    """In-place calls: the cache is restored (eagerly) before every replay."""
    g = W.kv_geometry(1)
    L, H, D, B, k, n, E, C = (g[x] for x in ("L", "H", "D", "B", "k", "n", "E", "C"))
    L = 2
    kv = torch.empty((L, 2, B, H, C, D), dtype=torch.bfloat16, device=DEV)
    W.fill_kv_torch(kv, E, n, torch.as_tensor(W.prefix_tokens(1, B, E + 1)).to(DEV), "bf16")
    orig = kv.clone()
    e = i32(np.random.default_rng(3).integers(1, k + 2, B))
    end = torch.tensor([E], dtype=torch.int32, device=DEV)
    nn = i32(n)
    outs = [torch.empty(1, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
            torch.empty(B, C, dtype=torch.int32, device=DEV), torch.empty(B, C, dtype=torch.int32, device=DEV),
            torch.empty(1, dtype=torch.int64, device=DEV)]

    def commit():
        sv.spec_commit_realign_kv(kv, k, end, nn, e, outs[0], outs[1], outs[2], outs[3], bytes_moved=outs[4])

    note("graph: commit realign")
    commit()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs] + [kv.clone()]
    g_ = torch.cuda.CUDAGraph()
    kv.copy_(orig)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        commit()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g_):
        commit()
    for rep in range(3):
        kv.copy_(orig)
        for o in outs:
            o.fill_(-7)
        torch.cuda.synchronize()
        g_.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs + [kv], want):
            assert torch.equal(o, w), rep


@pytest.mark.parametrize("c", [0, 2])
def test_rounds_of_verify_and_commit_replay(c):
    """Several rounds of verification and the realigning commit, chained on
    the device (each round's end column and lengths feed the next), captured
    in one graph from the initial state: every replay, after an eager reset of
    the cache, the end column and the lengths, leaves exactly what the eager
    rounds leave."""
    cfg = W.workload(c)
    R = 4
    g = W.kv_geometry(c, rounds=R)
    L, H, D, B, k, n, E, C = (g[x] for x in ("L", "H", "D", "B", "k", "n", "E", "C"))
    V = cfg["V"]
    kvdt = g["dtype"]
    note(f"graph: {R} rounds of verify + commit, workload {c} (B={B} k={k} V={V})")
    kv = torch.empty((L, 2, B, H, C, D), dtype=torch.bfloat16 if kvdt == "bf16" else torch.float32, device=DEV)
    tokens = torch.as_tensor(W.prefix_tokens(c, B, E + 1), device=DEV)
    i32e = dict(dtype=torch.int32, device=DEV)
    acc, emit, toks, offs = (torch.empty(B, **i32e), torch.empty(B, **i32e), torch.empty(B, k + 1, **i32e),
                             torch.empty(B + 1, **i32e))
    if cfg["mode"] == "greedy":
        rounds = [W.greedy_round(c, round_=r) for r in range(R)]
        ins = [(logits_to_device(r["logits"], r["dtype"]), i32(r["drafts"])) for r in rounds]
        dt = sv.SPEC_BF16 if rounds[0]["dtype"] == "bf16" else sv.SPEC_F32
        ws = sv.workspace(sv.spec_verify_greedy_workspace_bytes(B, k, V, dt), DEV)

        def verify(r):
            z, d = ins[r]
            sv.spec_verify_greedy(z, d, acc, emit, toks, ws, emit_offsets=offs)
    else:
        rounds = [W.sample_round(c, round_=r) for r in range(R)]
        ins = [tuple(torch.from_numpy(r[x]).to(DEV) for x in ("p", "q", "drafts", "uniforms")) for r in rounds]
        ws = sv.workspace(sv.spec_verify_sample_workspace_bytes(B, k, V), DEV)

        def verify(r):
            p_, q_, d, u = ins[r]
            sv.spec_verify_sample(p_, q_, d, u, acc, emit, toks, ws, emit_offsets=offs)
    Eb = [torch.empty(1, **i32e), torch.empty(1, **i32e)]
    Nb = [torch.empty(B, **i32e), torch.empty(B, **i32e)]
    pos, mask = torch.empty(B, C, **i32e), torch.empty(B, C, **i32e)

    def reset():
        W.fill_kv_torch(kv, E, n, tokens, kvdt)
        Eb[0].fill_(E)
        Nb[0].copy_(torch.as_tensor(n, **i32e))

    def run_rounds():
        for r in range(R):
            verify(r)
            sv.spec_commit_realign_kv(kv, k, Eb[r % 2], Nb[r % 2], emit, Eb[(r + 1) % 2], Nb[(r + 1) % 2],
                                      pos, mask)

    def state():
        return (kv, Eb[R % 2], Nb[R % 2], pos, mask, toks, emit, offs)

    reset()
    run_rounds()
    torch.cuda.synchronize()
    want = [x.clone() for x in state()]
    assert int(want[1].item()) > E                  # the rounds moved the end column
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_rounds()
    for rep in range(2):
        reset()
        toks.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(state(), want):
            assert torch.equal(a, b), rep
