"""Seeded synthetic inputs for the verify-and-commit step.

This module is the only code that both the CPU oracle and the GPU path use.
It builds inputs (logits, probability rows, draft tokens, uniforms, prefix
lengths, KV-cache contents) and holds none of the arithmetic of the method
itself: no acceptance decision, no residual, no realignment.

Everything is drawn from numpy's Philox bit generator, keyed by
(workload id, stream id, round, batch), so any process regenerates the same
bits.
"""
from .configs import (  # noqa: F401
    WORKLOADS,
    workload,
    stream,
    prefix_lengths,
    alphas,
    bf16_bits_from_f32,
    planted_greedy,
    random_tree,
    planted_tree,
    sampled_tree,
    greedy_round,
    sample_round,
    sample_logits,
    accept_counts,
    draw_inverse_cdf,
    kv_geometry,
    prefix_tokens,
    pool_lengths,
    policy_pool,
    policy_round,
)
from .kvfill import (  # noqa: F401
    kv_bits_np,
    kv_bits_torch,
    fill_kv_np,
    fill_kv_torch,
    write_forward_slots_np,
    write_forward_slots_torch,
    write_rows_np,
    write_rows_torch,
    KV_PAD_POS,
)
