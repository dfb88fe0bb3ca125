"""GPU parity of the paged-layout commit (spec_commit_paged) against the
oracle: every output is integer bookkeeping and must match exactly."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._gpu import commit_paged, host, logits_to_device, note, requires_gpu, verify_greedy

pytestmark = [pytest.mark.gpu, requires_gpu]


def _compare(k, page, n, e, bt):
    ref = oracle.commit_paged(n, e, k, page, bt)
    got = host(commit_paged(k, page, n, e, bt))
    assert np.array_equal(got["kv_len"], ref["kv_len"])
    assert np.array_equal(got["pages_kept"], ref["pages_kept"])
    assert np.array_equal(got["status"], ref["status"])
    assert np.array_equal(got["freed_offsets"], ref["freed_offsets"])
    nf = int(ref["freed_offsets"][-1])
    assert np.array_equal(got["freed"][:nf], ref["freed"])
    assert (got["freed"][nf:] == -7).all()                      # nothing written past the list


def _table(rng, B, max_pages):
    return rng.permutation(B * max_pages * 2)[:B * max_pages].reshape(B, max_pages).astype(np.int32)


def test_paged_random():
    rng = np.random.default_rng(31)
    for it in range(80):
        B, k = int(rng.integers(1, 40)), int(rng.integers(1, 12))
        page = int(rng.choice([1, 2, 3, 8, 16, 64, 256]))
        n = rng.integers(0, 600, B)
        max_pages = int(-(-(int(n.max()) + k + 1) // page)) + int(rng.integers(0, 3))
        e = rng.integers(0, k + 2, B)
        note(f"paged random {it}: B={B} k={k} page={page}")
        _compare(k, page, n, e, _table(rng, B, max_pages))


def test_paged_large_batch_and_invalid_rows():
    rng = np.random.default_rng(32)
    B, k, page = 5000, 8, 16
    n = rng.integers(0, 4000, B)
    e = rng.integers(0, k + 2, B)
    e[::97] = k + 5                                              # bad state
    n[5::101] = -3
    max_pages = 250
    n[7::89] = max_pages * page                                  # no room for the forward slots
    note("paged B=5000 with invalid rows")
    _compare(k, page, n, e, _table(rng, B, max_pages))


def test_paged_after_gpu_verification():
    rng = np.random.default_rng(33)
    B, k, V, page = 16, 6, 5000, 16
    g = W.planted_greedy(rng, rng, B, k, V, 1.0, "f32", rng.uniform(0.2, 1.0, B))
    note("paged after verify")
    e = host(verify_greedy(logits_to_device(g["logits"], "f32"), g["drafts"]))["emit_count"]
    n = rng.integers(0, 300, B)
    _compare(k, page, n, e, _table(rng, B, 40))
