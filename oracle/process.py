"""Processed sampling distributions from raw logits (oracle).  TEST
INFRASTRUCTURE ONLY.

[Walkthrough] 5.1 requires p and q to be the distributions actually sampled
from: when temperature, top-k or top-p is applied, the processed
probabilities are the ones compared in a(x) = min(1, p(x)/q(x)) and drawn
from.  The pages do not define the three operations; this oracle takes their
usual definitions, applied in the order temperature, top-k, top-p (readings,
listed in the design notes):

  * temperature T > 0: weight w(v) = exp((z(v) - max z) / T); a logit of -inf
    has weight 0;
  * top-k (K >= 1; 0 or K >= V = off): keep v when z(v) is at least the K-th
    largest logit of the row, counting repeats, so ties at the boundary are
    all kept;
  * top-p (0 < top_p < 1; 1 = off), over the entries kept by top-k: keep v
    when the total weight of the kept entries whose logit is strictly larger
    than z(v) is below top_p times the total kept weight.  This is the
    smallest top set whose mass reaches top_p, with ties at its boundary kept;
  * p'(v) = w(v) / (sum of the kept weights), rounded once to float32; dropped
    entries get 0; a row with no weight at all gets all zeros.

Arithmetic: logits are widened exactly to float64, T is the float32 value
widened to float64 and weights are float64.  The normalising sum is correctly
rounded (math.fsum); the top-p comparison is exact (integer arithmetic on the
float64 weights); top_p is the float32 value.  The kept sets are found by
sorting the logits, not by any selection algorithm.
"""
from __future__ import annotations

import math

import numpy as np


def _weights(z64: np.ndarray, zmax: float, T: float) -> np.ndarray:
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.exp((z64 - zmax) / T)
    return np.where(z64 == -np.inf, 0.0, w)


def top_k_keep(z64: np.ndarray, top_k: int) -> np.ndarray:
    """Mask of the entries whose logit is at least the K-th largest."""
    V = z64.size
    if top_k <= 0 or top_k >= V:
        return np.ones(V, bool)
    tau = np.sort(z64)[::-1][top_k - 1]
    return z64 >= tau


def _exact(x: float, scale_bits: int = 1200) -> int:
    """x (a non-negative float64) times 2**scale_bits, as an exact integer."""
    num, den = float(x).as_integer_ratio()
    return num << (scale_bits - (den.bit_length() - 1))


def top_p_keep(z64: np.ndarray, w: np.ndarray, kept: np.ndarray, top_p: float) -> np.ndarray:
    """Mask of the entries kept by top-p among `kept` (weights w).

    The weight sums and the comparison with top_p times the total are done
    exactly (integers scaled by 2**1200), so the kept set is the exact one for
    the float64 weights.
    """
    if top_p >= 1.0:
        return kept.copy()
    vals, inv = np.unique(z64[kept], return_inverse=True)      # distinct kept logits, ascending
    per = [0] * vals.size                                        # exact weight at each distinct logit
    for x, g in zip(w[kept].tolist(), inv.tolist()):
        per[g] += _exact(x)
    total = sum(per)
    num, den = float(np.float32(top_p)).as_integer_ratio()      # top_p = num / den exactly
    keep_val = np.zeros(vals.size, bool)
    above = 0                                                    # exact weight strictly above
    for i in range(vals.size - 1, -1, -1):
        keep_val[i] = above * den < num * total
        above += per[i]
    theta = vals[keep_val].min()
    return kept & (z64 >= theta)


def process_row(z, temperature: float, top_k: int = 0, top_p: float = 1.0):
    """(p' float32 [V], info) for one row of logits z (float32 or bf16-widened).

    info: zmax (float64), threshold (the smallest kept logit, or -inf when the
    row has no weight), mass (the kept weight, float64) and kept (bool mask).
    """
    z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
    V = z64.size
    T = float(np.float32(temperature))
    zmax = float(z64.max())
    if zmax == -np.inf:
        return np.zeros(V, np.float32), dict(zmax=zmax, threshold=-np.inf, mass=0.0,
                                             kept=np.ones(V, bool))
    kept = top_k_keep(z64, top_k)
    w = np.where(kept, _weights(z64, zmax, T), 0.0)
    kept = top_p_keep(z64, w, kept, top_p)
    w = np.where(kept, w, 0.0)
    mass = math.fsum(w)
    if not mass > 0.0:
        return np.zeros(V, np.float32), dict(zmax=zmax, threshold=float(z64[kept].min()),
                                             mass=mass, kept=kept)
    p = (w / mass).astype(np.float32)
    return p, dict(zmax=zmax, threshold=float(z64[kept].min()), mass=mass, kept=kept)


def process_rows(z: np.ndarray, temperature: float, top_k: int = 0, top_p: float = 1.0):
    """Apply process_row to every row of z [..., V]; returns (p' float32, list of info)."""
    shape = z.shape
    flat = z.reshape(-1, shape[-1])
    out = np.empty(flat.shape, np.float32)
    infos = []
    for r in range(flat.shape[0]):
        out[r], info = process_row(flat[r], temperature, top_k, top_p)
        infos.append(info)
    return out.reshape(shape), infos


def sample_verify_logits(zp: np.ndarray, zq: np.ndarray, drafts: np.ndarray, uniforms: np.ndarray,
                         temperature: float, top_k: int = 0, top_p: float = 1.0,
                         eos_id: int = -1, remaining=None) -> dict:
    """Stochastic verification on processed distributions: p' from the target
    logits zp [B, k+1, V], q' from the draft logits zq [B, k, V], then the
    verification of the stochastic oracle on (p', q')."""
    from .sample import sample_verify
    p, _ = process_rows(zp, temperature, top_k, top_p)
    q, _ = process_rows(zq, temperature, top_k, top_p)
    return sample_verify(p, q, drafts, uniforms, eos_id=eos_id, remaining=remaining)
