"""CPU oracle for the verify-and-commit step of batch speculative decoding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only the tests, the smoke entry point and the CPU
baseline leg of the benchmark do.  It is plain, slow, single-threaded
Python + numpy, written from the method's description and sharing no code,
constants or tables with the GPU library.

Sources (web pages, cited by title and section):
  [Forensics]  "Correctness Forensics for Batch Speculative Decoding:
               Diagnosing the Ragged Tensor Problem" (paperlayer.ai summary of
               arXiv 2510.22876v4): section 3 (EQSPEC invariants), 3.2 (EXSPEC
               same-length grouping), App. B (realignment), App. D (BatchVerify).
  [Walkthrough] zero-to-sglang "Chapter 10 Speculative Decoding (Code
               Walkthrough)": 3.3 (row alignment table), 4.1 (greedy commit),
               4.2 (worked rejection), 5.1 (acceptance and positive residual),
               5.2 (cache boundaries).
  [Design]     speculative-decoding-real "Design Document": Standard Greedy
               Algorithm, Key Property.
  [Atlas]      "Speculative decoding: proposals and verified output" (Atlas
               lesson): The mechanism; Acceptance and rejection correction;
               Output count in the iid acceptance scenario; Engineering example.

Pins (what ties each function to something other than itself) live in
tests/test_oracle_*.py.  Functions without such a pin say so here:
  group_same_length -- parity unpinned against the paper's own scheduler
  (its algorithm body is not on the page); pinned only by properties and
  brute force.  The EXSPEC loop (policy.py) inherits that: its grouping is
  this reading, and its pins are the per-sequence invariants.
"""
from .status import (  # noqa: F401
    ST_DRAFT_OOR, ST_Q_ZERO, ST_RESID_ZERO, ST_NONFINITE, ST_BAD_STATE, ST_CAPACITY,
)
from .greedy import (  # noqa: F401
    widen_bf16, argmax_first, greedy_commit, greedy_verify, verification_rows,
)
from .sample import accept_probability, draw_from_mass, sample_verify  # noqa: F401
from .process import process_row, process_rows, sample_verify_logits  # noqa: F401
from .realign import commit_bookkeeping, position_and_mask, commit_realign, resync_draft  # noqa: F401
from .group import group_same_length  # noqa: F401
from .paged import commit_paged  # noqa: F401
from .tree import tree_verify, compact_tree_slots  # noqa: F401
from .tree_sample import tree_sample_verify  # noqa: F401
from .unbatched import UnbatchedModel, check_ragged  # noqa: F401
from .ragged import repad_kv, unpad_kv, ragged_bytes  # noqa: F401
from .policy import eqspec_round, exspec_round  # noqa: F401
