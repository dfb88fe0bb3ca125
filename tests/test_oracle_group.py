"""Properties of the same-length grouping oracle.  Its parity with the
paper's own scheduler is unpinned (that algorithm's body is not on the page);
these tests pin the stated reading by properties and by brute force on tiny
pools."""
import itertools
from collections import Counter

import numpy as np
import pytest

import oracle
from workloads import pool_lengths


def _check(lengths, B, min_group, res):
    N = len(lengths)
    perm = res["perm"].tolist()
    assert sorted(perm) == list(range(N))                       # a partition of the window
    starts = res["batch_start"].tolist()
    assert starts[0] == 0 and starts[-1] == N and res["num_batches"] == len(starts) - 1
    blen = res["batch_len"].tolist()
    seen_mixed = False
    grouped = 0
    prev_len = -1
    for t in range(res["num_batches"]):
        members = perm[starts[t]:starts[t + 1]]
        assert 1 <= len(members) <= B
        assert members == sorted(members, key=lambda i: (lengths[i], i))
        if blen[t] >= 0:
            assert not seen_mixed                                 # uniform batches first
            assert all(lengths[i] == blen[t] for i in members)
            assert len(members) == B or len(members) >= min_group
            assert blen[t] >= prev_len
            prev_len = blen[t]
            grouped += len(members)
        else:
            seen_mixed = True
    assert res["num_grouped"] == grouped
    # per length: floor(c/B) full batches, plus one if the remainder reaches min_group
    cnt = Counter(lengths)
    per_len = Counter(blen[t] for t in range(res["num_batches"]) if blen[t] >= 0)
    for ell, c in cnt.items():
        want = c // B + (1 if c % B >= min_group else 0)
        assert per_len.get(ell, 0) == want
    # mixed batches are full except possibly the last
    mixed = [starts[t + 1] - starts[t] for t in range(res["num_batches"]) if blen[t] < 0]
    assert all(m == B for m in mixed[:-1])


@pytest.mark.parametrize("B,min_group", [(1, 1), (2, 2), (3, 2), (4, 1), (8, 2), (8, 3)])
def test_properties_random_pools(B, min_group):
    rng = np.random.default_rng(B * 10 + min_group)
    for _ in range(50):
        N = int(rng.integers(0, 60))
        lengths = rng.integers(1, 12, size=N).tolist()
        _check(lengths, B, min_group, oracle.group_same_length(lengths, B, min_group))


def test_bruteforce_tiny_pools():
    """Every pool of up to 5 sequences over 3 lengths: the fallback set is exactly
    the sequences of runs whose remainder is below min_group, taken from the
    end of their run in index order."""
    for N in range(0, 6):
        for lengths in itertools.product([1, 2, 3], repeat=N):
            for B, mg in [(2, 2), (3, 2), (2, 1)]:
                res = oracle.group_same_length(list(lengths), B, mg)
                _check(list(lengths), B, mg, res)
                want_fb = []
                for ell in sorted(set(lengths)):
                    run = [i for i in range(N) if lengths[i] == ell]
                    rem = len(run) % B
                    if 0 < rem < mg:
                        want_fb += run[len(run) - rem:]
                got_fb = res["perm"][res["num_grouped"]:].tolist()
                assert got_fb == want_fb


def test_identical_lengths_all_grouped():
    res = oracle.group_same_length([7] * 64, 8, 2)
    assert res["num_grouped"] == 64 and res["num_batches"] == 8
    assert (res["batch_len"] == 7).all()


def test_empty_window():
    res = oracle.group_same_length([], 8, 2)
    assert res["num_batches"] == 0 and res["perm"].size == 0 and res["batch_start"].tolist() == [0]


def test_grouping_rate_falls_with_batch_size():
    """On the heterogeneous pool, when only full same-length batches count
    (min_group = B), doubling B never groups more sequences (forensics
    summary 4.3: the grouping rate falls as batch size grows)."""
    P = pool_lengths().tolist()
    rates = [oracle.group_same_length(P, B, B)["num_grouped"] / len(P) for B in (2, 4, 8, 16)]
    assert rates[0] > 0
    assert all(x >= y for x, y in zip(rates, rates[1:]))
    assert rates[-1] < rates[0]
