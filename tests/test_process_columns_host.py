"""Host check that the long-row processed-distribution GPU test
(test_gpu_process.py::test_process_whole_row_histograms_of_long_rows) uses rows
whose whole-row histogram columns overflow a 10-bit count.

The statistics kernel streams a row in 16-byte vectors; vector i goes to
thread i mod 1024, whose lane index (i mod 64) selects the histogram column,
and the top 8 bits of the float's order key select the bucket.  A column of
one bucket then receives up to about V/64 logits.  The simulation below counts
them for the test's rows and confirms both that some column passes 1023 (the
packed count+weight word would wrap there) and that the kernel's bound on a
column's logits is never exceeded."""
import numpy as np
import pytest

import oracle
import workloads as W

PACKED_MAX_COLUMN = 1023


def _order_key(z: np.ndarray) -> np.ndarray:
    u = np.where(z == 0.0, np.float32(0.0), z).astype(np.float32).view(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def _column_counts(z: np.ndarray, vec: int) -> np.ndarray:
    """[256 buckets, 64 columns] logits per histogram cell of an aligned row."""
    lane = (np.arange(z.size) // vec) % 64
    bucket = _order_key(z) >> 24
    counts = np.zeros((256, 64), np.int64)
    np.add.at(counts, (bucket, lane), 1)
    return counts


def _packed_allowed(V: int, vec: int) -> bool:
    """The kernel's condition for packing counts and weights in one word."""
    return 16 * ((V // vec + 1023) // 1024) * vec + 2 <= PACKED_MAX_COLUMN


@pytest.mark.parametrize("dtype,V", [("bf16", 256000), ("f32", 256000), ("bf16", 524288)])
def test_long_rows_overflow_a_ten_bit_count(dtype, V):
    rng = np.random.default_rng(V % 1000 + (1 if dtype == "bf16" else 0))
    z = (rng.standard_normal((3, V)) * 1.0).astype(np.float32)     # as _rows(rng, 3, V, dtype, sd=1.0)
    if dtype == "bf16":
        z = oracle.widen_bf16(W.bf16_bits_from_f32(z))
    vec = 8 if dtype == "bf16" else 4
    bound = 16 * ((V // vec + 1023) // 1024) * vec + 2
    worst = 0
    for r in range(3):
        c = _column_counts(z[r], vec)
        assert c.sum() == V
        assert c.sum(axis=0).max() <= bound               # every column within the kernel's bound
        worst = max(worst, int(c.max()))
    assert worst > PACKED_MAX_COLUMN                       # a 10-bit count would wrap on these rows
    assert not _packed_allowed(V, vec)                     # so the kernel takes separate passes


def test_packing_bound_is_safe_where_used():
    """Wherever the kernel packs, no column can receive more than 1023 logits,
    even when every logit of the row falls into one bucket."""
    for vec in (4, 8):
        for V in range(1, 70000, 37):
            if _packed_allowed(V, vec):
                per_thread = -(-(V // vec) // 1024)             # vectors per thread, rounded up
                assert 16 * per_thread * vec + 2 <= PACKED_MAX_COLUMN
        # the largest packed rows: every logit equal (one bucket)
        Vmax = max(V for V in range(1, 70000) if _packed_allowed(V, vec))
        c = _column_counts(np.zeros(Vmax, np.float32), vec)
        assert c.max() <= PACKED_MAX_COLUMN
