// Processed sampling distributions from raw logits: temperature, top-k,
// top-p (gfx950).
//
// The zero-to-sglang walkthrough ("Chapter 10 Speculative Decoding", 5.1)
// requires p and q to be the distributions actually sampled from, so when
// temperature, top-k or top-p is applied the processed probabilities are the
// ones compared and drawn from.  The usual definitions are used, in the order
// temperature, top-k, top-p:
//   * weight w(v) = exp((z(v) - max z) / T), 0 for a logit of -inf;
//   * top-k keeps v when z(v) is at least the K-th largest logit (ties at the
//     boundary kept);
//   * top-p keeps v (among the top-k survivors) when the weight of the kept
//     entries with a strictly larger logit is below top_p times their total;
//   * p'(v) = w(v) / (kept weight); 0 when dropped.
// Weights are float32 (expf), sums float64 in a fixed order, so results are
// reproducible run to run and agree with a float64 evaluation to a relative
// 1e-5 or better (the error of a weight grows with |z - max z| / T).
// Both truncations keep every logit at or above a threshold, so a row is
// described by three numbers: its maximum, the threshold (as an order key of
// float32 values) and the kept weight.
#pragma once

#include "common.h"

namespace specv {

struct ProcStats {
  float zmax;       // largest logit of the row (-inf when every logit is -inf)
  uint32_t theta;   // entry v is kept iff f32_order_key(z(v)) >= theta
  double mass;      // kept weight, float64 sum of the float32 weights; 0: no mass
  float inv_mass;   // 1 / mass rounded to float32 (0 when the row has no mass)
  float zmin_kept;  // smallest kept logit
};

int launch_proc_stats(const void *za, const void *zb, int rows_a, int rows, int V, bool bf16,
                      float T, int top_k, float top_p, ProcStats *stats, float *probs,
                      hipStream_t s);
bool proc_args_ok(float T, int top_k, float top_p, int V);

struct ProcConfig {
  float T;          // temperature > 0
  int top_k;        // 0 = off
  float top_p;      // >= 1 = off
};

template <bool BF16>
__device__ inline float logit_at(const void *row, int v) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(row)[v]) << 16);
  } else {
    return static_cast<const float *>(row)[v];
  }
}

// Weight exp((z - zmax) / T) in float32: one rounded subtraction (exact for
// bf16 logits of ordinary range), one IEEE division and expf.
__device__ inline float proc_weight(float z, float zmax, float T) {
  if (z == -INFINITY) return 0.0f;
  return expf(__fdiv_rn(z - zmax, T));
}

// Processed probability of one entry of a row with statistics s.
__device__ inline float proc_prob(float z, const ProcStats &s, float T) {
  if (!(s.mass > 0.0) || f32_order_key(z) < s.theta) return 0.0f;
  return proc_weight(z, s.zmax, T) * s.inv_mass;
}

}  // namespace specv
