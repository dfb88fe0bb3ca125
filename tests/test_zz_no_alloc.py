"""spec_verify_greedy_noalloc (no workspace, no allocation: the library's
static per-GPU array) against spec_verify_greedy through the C ABI: every
output bit-exact, on two calls in a row, the second with a smaller input, and
sizes beyond the array rejected."""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_04_amd as sv
import workloads as W
from tests._gpu import DEV, i32, logits_to_device, note, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

NAMES = ["accept_len", "emit_count", "out_tokens", "emit_offsets", "status"]


def _outputs(B, kp1):
    return {n: torch.full((B + 1,) if n == "emit_offsets" else ((B, kp1) if n == "out_tokens" else (B,)),
                          -77, dtype=torch.int32, device=DEV) for n in NAMES}


def _both(logits, drafts, eos_id=-1, remaining=None):
    B, kp1, V = logits.shape
    dt = sv.SPEC_BF16 if logits.dtype == torch.bfloat16 else sv.SPEC_F32
    ref, got = _outputs(B, kp1), _outputs(B, kp1)
    ws = sv.workspace(sv.spec_verify_greedy_workspace_bytes(B, kp1 - 1, V, dt), DEV)
    sv.spec_verify_greedy(logits, drafts, ref["accept_len"], ref["emit_count"], ref["out_tokens"], ws,
                          eos_id=eos_id, remaining=remaining, emit_offsets=ref["emit_offsets"], status=ref["status"])
    sv.spec_verify_greedy_noalloc(logits, drafts, got["accept_len"], got["emit_count"], got["out_tokens"],
                                  eos_id=eos_id, remaining=remaining, emit_offsets=got["emit_offsets"],
                                  status=got["status"])
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n
    return got


def test_noalloc_matches_greedy_verify_on_two_calls():
    # call 1: the large-batch workload (B=32, k=8, V=128256 bf16);
    # call 2, smaller: the mid-size workload (B=8, k=5, V=32000 bf16)
    for c in (3, 1):
        note(f"noalloc vs greedy, workload {c}")
        g = W.greedy_round(c, round_=2)
        x = logits_to_device(g["logits"], g["dtype"])
        got = _both(x, i32(g["drafts"]))
        assert int(got["emit_count"].min().item()) >= 1


def test_noalloc_eos_budget_and_bad_drafts():
    note("noalloc eos/budget/out-of-range drafts")
    rng = np.random.default_rng(4)
    B, k, V = 40, 6, 3000
    z = rng.standard_normal((B, k + 1, V)).astype(np.float32)
    amax = np.argmax(z, axis=-1)
    drafts = np.where(rng.random((B, k)) < 0.8, amax[:, :k], rng.integers(0, V, (B, k))).astype(np.int32)
    drafts[::5, 1] = V + 2
    rem = rng.integers(-1, k + 3, size=B).astype(np.int32)
    _both(logits_to_device(z, "f32"), i32(drafts), eos_id=int(amax[0, 2]), remaining=i32(rem))


def test_noalloc_rejects_sizes_beyond_its_array():
    note("noalloc capacity")
    B, k, V = 8193, 127, 1          # 8193 * 128 chunk results of 8 bytes: just over 8 MiB
    assert sv.spec_verify_greedy_workspace_bytes(B, k, V, sv.SPEC_F32) > sv.SPEC_GREEDY_SCRATCH_BYTES
    x = torch.zeros(B, k + 1, V, dtype=torch.float32, device=DEV)
    d = torch.zeros(B, k, dtype=torch.int32, device=DEV)
    o = _outputs(B, k + 1)
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_greedy_noalloc(x, d, o["accept_len"], o["emit_count"], o["out_tokens"])
    assert e.value.code == sv.SPEC_ECAPACITY
    assert int((o["emit_count"] == -77).sum().item()) == B          # nothing was launched
