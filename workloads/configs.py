"""The five synthetic workloads and their seeded generators.

Workload shapes follow the verify-and-commit workloads the method is stated
for: a batch of B sequences, k draft proposals each, a vocabulary of V ids,
a contiguous left-padded KV cache of L layers x {K,V} x H heads x head_dim D.
They stand in for the public benchmarks the pages measure on (SpecBench,
Multi30k), which are not reproduced here.

Conventions (readings of the workload descriptions):
  * "N(0, s)" means a normal with standard deviation s.
  * A sequence with prefix length P has P confirmed tokens; its KV cache
    holds P - 1 rows (the last confirmed token is not cached yet), and the
    verify forward appends k + 1 rows: the last confirmed token plus the k
    drafts.
  * Planted greedy drafts: per slot, independently, the draft equals the
    argmax of that target row with probability alpha_b, otherwise a uniform
    draw among the other V - 1 ids.  The argmax used here only shapes the
    acceptance rate; no parity result depends on it.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = [
    dict(id=0, name="tiny greedy verify+realign", mode="greedy",
         B=4, k=4, V=1000, logit_dtype="f32", logit_sd=1.0, alpha=(0.7, 0.7),
         kv_dtype="f32", L=2, H=4, D=64, prefix=(16, 64)),
    dict(id=1, name="greedy mid-size", mode="greedy",
         B=8, k=5, V=32000, logit_dtype="bf16", logit_sd=2.0, alpha=(0.5, 0.9),
         kv_dtype="bf16", L=24, H=16, D=64, prefix=(128, 1024)),
    dict(id=2, name="stochastic rejection sampling", mode="sample",
         B=8, k=4, V=151936, z_sd=3.0, temperature=0.7, eps_sd=1.0,
         kv_dtype="bf16", L=24, H=2, D=64, prefix=(256, 2048)),
    dict(id=3, name="large-batch greedy, realign-heavy", mode="greedy",
         B=32, k=8, V=128256, logit_dtype="bf16", logit_sd=2.0, alpha=(0.3, 0.95),
         kv_dtype="bf16", L=32, H=8, D=128, prefix=(512, 4096)),
    dict(id=4, name="grouped stochastic (same-length scheduling)", mode="grouped",
         pool=256, B=8, min_group=2, k=4, V=256000, z_sd=3.0, temperature=0.7,
         eps_sd=1.0, alpha=(0.4, 0.9), kv_dtype="bf16", L=28, H=4, D=128,
         prefix=(64, 2048), warm_rounds=8),
]

_STREAM_IDS = {
    "lengths": 1, "alpha": 2, "logits": 3, "drafts": 4, "uniforms": 5,
    "kv": 6, "tokens": 7, "eps": 8, "pool": 9, "accept": 10,
    "policy_logits": 11, "policy_drafts": 12, "tree": 13,
}


def workload(c: int) -> dict:
    return dict(WORKLOADS[c])


def stream(c: int, name: str, round_: int = 0, batch: int = 0) -> np.random.Generator:
    """Independent Philox stream for (workload, purpose, round, batch)."""
    ss = np.random.SeedSequence([1000 + int(c), _STREAM_IDS[name], int(round_), int(batch)])
    return np.random.Generator(np.random.Philox(ss))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _widen_for_planting(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def prefix_lengths(c: int, B: int | None = None) -> np.ndarray:
    cfg = WORKLOADS[c]
    n = cfg.get("pool", cfg["B"]) if B is None else B
    lo, hi = cfg["prefix"]
    return stream(c, "lengths").integers(lo, hi + 1, size=n).astype(np.int64)


def alphas(c: int, B: int | None = None) -> np.ndarray:
    cfg = WORKLOADS[c]
    n = cfg.get("pool", cfg["B"]) if B is None else B
    lo, hi = cfg["alpha"]
    return stream(c, "alpha").uniform(lo, hi, size=n)


def planted_greedy(g_logits: np.random.Generator, g_drafts: np.random.Generator,
                   B: int, k: int, V: int, sd: float, dtype: str, alpha) -> dict:
    """Logits [B, k+1, V] ~ N(0, sd) and drafts planted with per-sequence rate alpha.

    bf16 logits are returned as their uint16 bit patterns (numpy has no
    bfloat16); f32 logits as float32.
    """
    z = g_logits.standard_normal((B, k + 1, V), dtype=np.float32)
    z *= np.float32(sd)
    if dtype == "bf16":
        logits = bf16_bits_from_f32(z)
        view = _widen_for_planting(logits)
    else:
        logits = z
        view = z
    amax = np.argmax(view[:, :k, :], axis=-1)
    a = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (B,))
    plant = g_drafts.random((B, k)) < a[:, None]
    other = g_drafts.integers(0, V - 1, size=(B, k))
    other = other + (other >= amax)
    drafts = np.where(plant, amax, other).astype(np.int32)
    return dict(logits=logits, dtype=dtype, drafts=drafts, B=B, k=k, V=V)


def random_tree(rng: np.random.Generator, N: int, branching: int = 3):
    """A random tree of N nodes in topological order: node i's parent is drawn
    uniformly from the `branching` nodes just below i.  Returns the parent list
    and the first_child / next_sibling links (children in index order)."""
    parent = np.full(N, -1, np.int64)
    fc = np.full(N, -1, np.int32)
    ns = np.full(N, -1, np.int32)
    last = np.full(N, -1, np.int64)
    for i in range(1, N):
        p = int(rng.integers(max(0, i - branching), i))
        parent[i] = p
        if fc[p] == -1:
            fc[p] = i
        else:
            ns[last[p]] = i
        last[p] = i
    return parent, fc, ns


def planted_tree(g_logits: np.random.Generator, g_drafts: np.random.Generator,
                 B: int, N: int, V: int, sd: float, dtype: str, alpha, branching: int = 3) -> dict:
    """A candidate tree per sequence with logits [B, N, V] ~ N(0, sd).

    Node i > 0 proposes, with probability alpha_b, the argmax of its parent's
    row (so siblings may propose the same id), else a uniform id other than
    it; draft[b, 0] is 0.  As in planted_greedy the argmax only shapes how deep
    verification goes.  bf16 logits are returned as uint16 bits."""
    z = g_logits.standard_normal((B, N, V), dtype=np.float32)
    z *= np.float32(sd)
    if dtype == "bf16":
        logits = bf16_bits_from_f32(z)
        view = _widen_for_planting(logits)
    else:
        logits = z
        view = z
    amax = np.argmax(view, axis=-1)
    a = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (B,))
    parent = np.full((B, N), -1, np.int64)
    fc = np.full((B, N), -1, np.int32)
    ns = np.full((B, N), -1, np.int32)
    draft = np.zeros((B, N), np.int32)
    for b in range(B):
        parent[b], fc[b], ns[b] = random_tree(g_drafts, N, branching)
        for i in range(1, N):
            want = int(amax[b, parent[b, i]])
            if g_drafts.random() < a[b]:
                draft[b, i] = want
            else:
                o = int(g_drafts.integers(0, V - 1))
                draft[b, i] = o + (o >= want)
    return dict(logits=logits, dtype=dtype, draft=draft, first_child=fc, next_sibling=ns,
                parent=parent, B=B, N=N, V=V)


def greedy_round(c: int, round_: int = 0, B: int | None = None) -> dict:
    """Target logits and planted drafts of workload c for one verify round."""
    cfg = WORKLOADS[c]
    B = cfg["B"] if B is None else B
    return planted_greedy(stream(c, "logits", round_), stream(c, "drafts", round_),
                          B, cfg["k"], cfg["V"], cfg["logit_sd"], cfg["logit_dtype"],
                          alphas(c, B))


def _softmax_f32(x64: np.ndarray) -> np.ndarray:
    m = x64.max(axis=-1, keepdims=True)
    e = np.exp(x64 - m)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def sample_round(c: int, round_: int = 0, batch: int = 0, B: int | None = None,
                 V: int | None = None, k: int | None = None) -> dict:
    """Target rows p [B, k+1, V], draft rows q [B, k, V] (float32), drafts x ~ q,
    and uniforms [B, k+1] (float32 in [0, 1)).

    p = softmax(z / T), q = softmax((z + eps) / T), z ~ N(0, z_sd), eps ~ N(0, eps_sd).
    """
    cfg = WORKLOADS[c]
    B = cfg["B"] if B is None else B
    k = cfg["k"] if k is None else k
    V = cfg["V"] if V is None else V
    T = cfg["temperature"]
    z = stream(c, "logits", round_, batch).standard_normal((B, k + 1, V), dtype=np.float32)
    z *= np.float32(cfg["z_sd"])
    eps = stream(c, "eps", round_, batch).standard_normal((B, k, V), dtype=np.float32)
    eps *= np.float32(cfg["eps_sd"])
    p = _softmax_f32(z.astype(np.float64) / T)
    q = _softmax_f32((z[:, :k].astype(np.float64) + eps.astype(np.float64)) / T)
    del z, eps
    # Drafting is outside the step under test: draw x ~ q by inverse CDF.
    ud = stream(c, "drafts", round_, batch).random((B, k))
    drafts = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        for j in range(k):
            cq = np.cumsum(q[b, j].astype(np.float64))
            x = int(np.searchsorted(cq, ud[b, j] * cq[-1], side="right"))
            drafts[b, j] = min(x, V - 1)
    u = stream(c, "uniforms", round_, batch).random((B, k + 1), dtype=np.float32)
    return dict(p=p, q=q, drafts=drafts, uniforms=u, B=B, k=k, V=V)


def sampled_tree(rng: np.random.Generator, B: int, N: int, V: int, z_sd: float = 3.0, eps_sd: float = 1.0,
                 temperature: float = 0.7, branching: int = 3) -> dict:
    """Candidate trees for stochastic tree verification: per sequence a
    random_tree of N nodes; per node a target row p = softmax(z / T) and a
    draft row q = softmax((z + eps) / T) (z ~ N(0, z_sd), eps ~ N(0, eps_sd),
    float32); node c > 0 proposes an id drawn from q of its parent by inverse
    CDF (drafting, outside the step under test), so siblings are independent
    draws; uniforms [B, N] float32 in [0, 1)."""
    z = rng.standard_normal((B, N, V), dtype=np.float32)
    z *= np.float32(z_sd)
    eps = rng.standard_normal((B, N, V), dtype=np.float32)
    eps *= np.float32(eps_sd)
    p = _softmax_f32(z.astype(np.float64) / temperature)
    q = _softmax_f32((z.astype(np.float64) + eps.astype(np.float64)) / temperature)
    del z, eps
    fc = np.full((B, N), -1, np.int32)
    ns = np.full((B, N), -1, np.int32)
    draft = np.zeros((B, N), np.int32)
    ud = rng.random((B, N))
    for b in range(B):
        parent, fc[b], ns[b] = random_tree(rng, N, branching)
        for c in range(1, N):
            cq = np.cumsum(q[b, parent[c]].astype(np.float64))
            draft[b, c] = min(int(np.searchsorted(cq, ud[b, c] * cq[-1], side="right")), V - 1)
    u = rng.random((B, N), dtype=np.float32)
    return dict(p=p, q=q, draft=draft, first_child=fc, next_sibling=ns, uniforms=u, B=B, N=N, V=V)


def sample_logits(c: int, round_: int = 0, batch: int = 0, B: int | None = None,
                  V: int | None = None, k: int | None = None) -> dict:
    """Raw logits of the stochastic workloads before any processing: target
    logits z [B, k+1, V] and draft logits z[:, :k] + eps [B, k, V] (float32),
    from the same streams as sample_round, plus its uniforms [B, k+1]."""
    cfg = WORKLOADS[c]
    B = cfg["B"] if B is None else B
    k = cfg["k"] if k is None else k
    V = cfg["V"] if V is None else V
    z = stream(c, "logits", round_, batch).standard_normal((B, k + 1, V), dtype=np.float32)
    z *= np.float32(cfg["z_sd"])
    eps = stream(c, "eps", round_, batch).standard_normal((B, k, V), dtype=np.float32)
    eps *= np.float32(cfg["eps_sd"])
    zd = z[:, :k] + eps
    u = stream(c, "uniforms", round_, batch).random((B, k + 1), dtype=np.float32)
    return dict(zt=z, zd=zd, uniforms=u, B=B, k=k, V=V, temperature=cfg["temperature"])


def draw_inverse_cdf(probs: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Ids drawn from the rows of probs [..., V] by inverse CDF with uniforms u [...]
    (drafting, outside the step under test)."""
    flat = probs.reshape(-1, probs.shape[-1]).astype(np.float64)
    uf = np.asarray(u, np.float64).reshape(-1)
    out = np.empty(flat.shape[0], np.int32)
    for r in range(flat.shape[0]):
        c = np.cumsum(flat[r])
        out[r] = min(int(np.searchsorted(c, uf[r] * c[-1], side="right")), flat.shape[1] - 1)
    return out.reshape(probs.shape[:-1])


def accept_counts(c: int, round_: int, B: int | None = None) -> np.ndarray:
    """Emitted counts e_b of one synthetic round (inputs for commit-only runs):
    e_b - 1 is the number of leading successes among k iid trials of
    probability alpha_b (the planted-draft law), so e_b is in 1..k+1."""
    cfg = WORKLOADS[c]
    B = cfg["B"] if B is None else B
    k = cfg["k"]
    a = alphas(c, B)
    trials = stream(c, "accept", round_).random((B, k)) < a[:, None]
    lead = np.argmin(np.concatenate([trials, np.zeros((B, 1), bool)], axis=1), axis=1)
    return (lead + 1).astype(np.int32)


def kv_geometry(c: int, rounds: int = 1, B: int | None = None) -> dict:
    """Shape of the left-padded rectangle: n_b cached rows, end column E, capacity C.

    C = E + (k + 1) * rounds leaves room for `rounds` verify forwards.
    """
    cfg = WORKLOADS[c]
    B = cfg["B"] if B is None else B
    P = prefix_lengths(c, B)
    n = P - 1
    E = int(n.max())
    k = cfg["k"]
    return dict(L=cfg["L"], H=cfg["H"], D=cfg["D"], B=B, k=k, dtype=cfg["kv_dtype"],
                n=n.astype(np.int64), E=E, C=E + (k + 1) * rounds)


def prefix_tokens(c: int, B: int, length: int, V: int | None = None) -> np.ndarray:
    """Synthetic confirmed tokens [B, length] (ids in [0, V))."""
    V = WORKLOADS[c]["V"] if V is None else V
    return stream(c, "tokens").integers(0, V, size=(B, length)).astype(np.int64)


def pool_lengths(c: int = 4) -> np.ndarray:
    """Prefix lengths of the same-length-scheduling pool after its warm-up rounds.

    Each warm-up round every sequence gains e tokens, where e - 1 is the number
    of leading successes among k iid trials of probability alpha_b (so e is in
    1..k+1), which makes the pool's lengths drift apart as they would under
    verification.
    """
    cfg = WORKLOADS[c]
    P = prefix_lengths(c).copy()
    a = alphas(c)
    k = cfg["k"]
    g = stream(c, "pool")
    for _ in range(cfg.get("warm_rounds", 0)):
        trials = g.random((P.size, k)) < a[:, None]
        lead = np.argmin(np.concatenate([trials, np.zeros((P.size, 1), bool)], axis=1), axis=1)
        P = P + lead + 1
    return P.astype(np.int64)


def policy_pool(kind: str = "drifted") -> dict:
    """Pool of the multi-round scheduling comparison (the grouped workload's
    256 sequences, their acceptance rates, k = 4 drafts, batches of 8).

    drifted: the grouped workload's pool after its warm-up rounds (lengths
             spread over about 2000 values);
    four:    the same sequences with lengths drawn from four values, a
             homogeneous workload.
    P holds confirmed-token counts; the caches hold P - 1 rows."""
    cfg = WORKLOADS[4]
    P = pool_lengths(4)
    if kind == "four":
        P = stream(4, "pool", 99).choice(np.array([512, 513, 900, 1500]), size=P.size)
    elif kind != "drifted":
        raise ValueError(kind)
    return dict(P=P.astype(np.int64), alpha=alphas(4), k=cfg["k"], B=cfg["B"], min_group=cfg["min_group"],
                N=int(P.size))


def policy_round(r: int, N: int, k: int, V: int, dtype: str, sd: float, alpha) -> dict:
    """Greedy verification inputs of every pool sequence for round r: sequence
    s gets logits [k+1, V] ~ N(0, sd) and drafts planted with alpha[s] from
    its own streams, so the inputs do not depend on how sequences are
    batched."""
    logits = np.empty((N, k + 1, V), np.uint16 if dtype == "bf16" else np.float32)
    drafts = np.empty((N, k), np.int32)
    for s in range(N):
        g = planted_greedy(stream(4, "policy_logits", r, s), stream(4, "policy_drafts", r, s), 1, k, V, sd,
                           dtype, np.asarray(alpha)[s:s + 1])
        logits[s] = g["logits"][0]
        drafts[s] = g["drafts"][0]
    return dict(logits=logits, drafts=drafts, dtype=dtype)
