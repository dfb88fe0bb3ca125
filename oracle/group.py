"""Same-length grouping of a pool of ragged sequences (oracle).
TEST INFRASTRUCTURE ONLY.

[Forensics] 3.2 describes EXSPEC: keep sequences ragged, form batches of
identical-length sequences from a sliding window larger than the batch size,
and fall back to unpad-append-repad when no group forms.  The algorithm body
(App. C) is not on the page, so this function is a reading and its parity
with the paper's scheduler is UNPINNED; the tests pin it by properties and
brute force only.

Reading:
  1. the window is the whole lengths array passed in;
  2. order indices by (length, index);
  3. walk the equal-length runs in ascending length; cut each run into
     floor(count / B) full batches; a remainder of at least min_group
     sequences becomes one more (smaller) same-length batch, a smaller
     remainder goes to the fallback list in (length, index) order;
  4. cut the fallback list into mixed batches of B (the last may be short);
  5. same-length batches come first, then mixed ones.
Outputs: perm (the window indices in batch order), batch_start [nb + 1],
batch_len [nb] (the shared length, or -1 for a mixed batch), and the number
of sequences placed in same-length batches.
"""
from __future__ import annotations

import numpy as np


def group_same_length(lengths, B: int, min_group: int = 2) -> dict:
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    order = sorted(range(N), key=lambda i: (lengths[i], i))
    uniform = []
    fallback = []
    i = 0
    while i < N:
        j = i
        while j < N and lengths[order[j]] == lengths[order[i]]:
            j += 1
        run = order[i:j]
        full = len(run) // B
        for t in range(full):
            uniform.append(run[t * B:(t + 1) * B])
        rest = run[full * B:]
        if len(rest) >= min_group:
            uniform.append(rest)
        else:
            fallback.extend(rest)
        i = j
    mixed = [fallback[t:t + B] for t in range(0, len(fallback), B)]
    batches = uniform + mixed
    perm = np.array([x for bt in batches for x in bt], np.int32)
    batch_start = np.zeros(len(batches) + 1, np.int32)
    for t, bt in enumerate(batches):
        batch_start[t + 1] = batch_start[t] + len(bt)
    batch_len = np.array([lengths[bt[0]] for bt in uniform] + [-1] * len(mixed), np.int32)
    return dict(perm=perm, batch_start=batch_start, batch_len=batch_len,
                num_batches=len(batches), num_grouped=int(sum(len(bt) for bt in uniform)))
