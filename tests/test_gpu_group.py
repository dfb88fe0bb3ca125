"""GPU parity of spec_group_same_length (bit-exact against the oracle's
reading of same-length grouping), and the grouped stochastic workload end to
end: group the pool, verify each batch, commit same-length batches by a
length update and mixed batches by realignment."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import DEV, commit, group, host, kv_bits, note, requires_gpu, verify_sample

pytestmark = [pytest.mark.gpu, requires_gpu]


def _compare(lengths, B, mg):
    ref = oracle.group_same_length(lengths, B, mg)
    got = host(group(lengths, B, mg))
    nb = int(got["num_batches"][0])
    assert nb == ref["num_batches"]
    assert int(got["num_grouped"][0]) == ref["num_grouped"]
    N = len(lengths)
    assert np.array_equal(got["perm"][:N], ref["perm"])
    assert np.array_equal(got["batch_start"][:nb + 1], ref["batch_start"])
    assert np.array_equal(got["batch_len"][:nb], ref["batch_len"])
    return ref


def test_pool_workload():
    note("group workload 4 pool")
    P = W.pool_lengths()
    ref = _compare(P.tolist(), 8, 2)
    assert 0 < ref["num_grouped"] < len(P)


@pytest.mark.parametrize("N", [0, 1, 2, 17, 256, 1000, 4096])
@pytest.mark.parametrize("B,mg", [(1, 1), (3, 2), (8, 2), (8, 5), (32, 1)])
def test_random_windows(N, B, mg):
    note(f"group N={N} B={B} mg={mg}")
    rng = np.random.default_rng(N * 100 + B * 10 + mg)
    for spread in (4, 3000):
        lengths = rng.integers(-spread // 2, spread, size=N).tolist()
        _compare(lengths, B, mg)


@pytest.mark.parametrize("N", [63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 2047, 2049])
def test_sort_path_boundaries(N):
    """Windows on either side of the sort's limits: one key per lane up to
    1024 keys (lane shuffles below a wave), LDS above; lengths with many ties,
    and lengths spread over the whole int32 range."""
    note(f"group boundary N={N}")
    rng = np.random.default_rng(9000 + N)
    for B, mg in [(1, 1), (8, 2), (64, 8)]:
        _compare(rng.integers(0, 5, size=N).tolist(), B, mg)
        _compare(rng.integers(-2 ** 31, 2 ** 31 - 1, size=N, dtype=np.int64).tolist(), B, mg)


def test_all_equal_and_extremes():
    note("group extremes")
    _compare([5] * 4096, 8, 2)
    _compare([2 ** 31 - 1, -2 ** 31, 0, 2 ** 31 - 1, -2 ** 31], 2, 2)


def test_grouped_workload_end_to_end():
    """Workload 4: pool of 256, batches of up to 8, k=4, V=256000, KV 28 x 4 x 128 bf16."""
    c = 4
    cfg = W.workload(c)
    P = W.pool_lengths()
    note("grouped workload: grouping")
    gr = host(group(P.tolist(), cfg["B"], cfg["min_group"]))
    ref_g = oracle.group_same_length(P.tolist(), cfg["B"], cfg["min_group"])
    nb = int(gr["num_batches"][0])
    assert nb == ref_g["num_batches"] and np.array_equal(gr["perm"], ref_g["perm"])
    k, L, H, D = cfg["k"], cfg["L"], cfg["H"], cfg["D"]
    uniform = [t for t in range(nb) if gr["batch_len"][t] >= 0]
    mixed = [t for t in range(nb) if gr["batch_len"][t] < 0]
    rng = np.random.default_rng(44)
    for t in uniform[:2] + mixed[:1]:
        members = gr["perm"][gr["batch_start"][t]:gr["batch_start"][t + 1]]
        Bt = len(members)
        note(f"grouped workload: batch {t} ({'same-length' if gr['batch_len'][t] >= 0 else 'mixed'}, {Bt})")
        r = W.sample_round(c, batch=t, B=Bt)
        got = host(verify_sample(torch.from_numpy(r["p"]).to(DEV), torch.from_numpy(r["q"]).to(DEV),
                                 r["drafts"], r["uniforms"]))
        ref = oracle.sample_verify(r["p"], r["q"], r["drafts"], r["uniforms"])
        from tests.test_gpu_sample import check_within_tolerance
        ex, tol = check_within_tolerance(r["p"], r["q"], r["drafts"], r["uniforms"], got, ref)
        assert tol == 0 and ex == Bt
        n = P[members] - 1
        if gr["batch_len"][t] >= 0:
            # same-length batch: already rectangular, the commit is a length update
            assert (P[members] == gr["batch_len"][t]).all()
            continue
        # mixed batch: left-pad into a rectangle and realign on commit
        E = int(n.max())
        C = E + k + 1
        tokens = rng.integers(0, cfg["V"], (Bt, E + 1))
        kv = torch.empty((L, 2, Bt, H, C, D), dtype=torch.bfloat16, device=DEV)
        W.fill_kv_torch(kv, E, n, torch.as_tensor(tokens).to(DEV), "bf16")
        pre = kv_bits(kv)
        refc = oracle.commit_realign(pre, E, n, got["emit_count"], k)
        out = host(commit(kv, k, E, n, got["emit_count"]))
        assert np.array_equal(kv_bits(kv), refc["kv"])
        assert np.array_equal(out["pos"], refc["pos"]) and np.array_equal(out["mask"], refc["mask"])
        assert int(out["bytes_moved"][0]) == refc["bytes_moved"]
