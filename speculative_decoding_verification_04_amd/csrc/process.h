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
// Weights are float32: the accurate expf of (z - max z) / T, whose argument's
// rounding error is folded back in to first order, so a weight is within a
// few float32 ulps of the exact one whatever |z - max z| / T is; sums are
// exact integer sums of the weights truncated to 2^-40, so results are
// reproducible run to run.
// Both truncations keep every logit at or above a threshold, so a row is
// described by three numbers: its maximum, the threshold (as an order key of
// float32 values) and the kept weight.
#pragma once

#include "common.h"

namespace specv {

// 1 / temperature: its float32 value and the exact residual 1 - T * inv
// (computed with one fma), so that (z - zmax) / T = (z - zmax) * inv * (1 + corr)
// up to corr^2 (|corr| <= 2^-24).
struct Temper {
  float inv;
  float corr;
};

__host__ __device__ inline Temper make_temper(float T) {
  Temper t;
  t.inv = 1.0f / T;
  t.corr = fmaf(-T, t.inv, 1.0f);
  return t;
}

struct ProcStats {
  float zmax;       // largest logit of the row (-inf when every logit is -inf)
  uint32_t theta;   // entry v is kept iff f32_order_key(z(v)) >= theta
  double mass;      // kept weight: exact sum of the weights in 2^-40 units; 0: no mass
  float inv_mass;   // 1 / mass rounded to float32 (0 when the row has no mass)
  float zmin_kept;  // smallest kept logit
};

// Statistics of rows [0, rows) (rows_a from za, the rest from zb) into stats;
// list_ws (proc_list_bytes(rows, V), or null to always read whole rows) holds
// the slice kernels' candidate lists and per-slice sums.
int launch_proc_stats(const void *za, const void *zb, int rows_a, int rows, int V, bool bf16,
                      Temper invT, int top_k, float top_p, ProcStats *stats, float *probs,
                      void *list_ws, hipStream_t s);
size_t proc_list_bytes(int rows, int V);
// Workspace of the slice lists' entry indices (the verification from logits).
size_t proc_list_idx_bytes(int rows);
bool proc_args_ok(float T, int top_k, float top_p, int V);

struct ProcConfig {
  Temper invT;      // 1 / temperature
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

// Weight exp((z - zmax) / T) in float32, with the argument carried beyond
// float32: d = z - zmax and its rounding error dl (TwoSum, exact; dl is 0 for
// bf16 logits of ordinary range); x = d * inv rounded, and
// c = (d * inv - x) + dl * inv + x * corr (the product's error by fma, the
// difference's error and the error of inv as 1/T), so that
// (z - zmax) / T = x + c up to about 2^-46 |x|.  The weight is expf(x) * (1 + c)
// with the accurate expf; c^2 / 2 is below 2^-40 for |x| < 100.  Relative error
// about 2^-23 + 2^-24 for every argument (a bare exponential of a rounded
// argument errs by about 2^-24 |x| instead).
__device__ inline float proc_weight(float z, float zmax, Temper tp) {
  if (z == -INFINITY) return 0.0f;
  const float d = z - zmax;
  const float bb = d - z;
  const float dl = (z - (d - bb)) + (-zmax - bb);
  const float x = d * tp.inv;
  const float c = fmaf(x, tp.corr, fmaf(dl, tp.inv, fmaf(d, tp.inv, -x)));
  const float e = expf(x);
  return fmaf(e, c, e);
}

// A weight in [0, 1] as an integer number of 2^-40 units (truncated):
// floor(w * 2^40) = floor(w * 2^20) * 2^20 + floor(frac(w * 2^20) * 2^20),
// where each product by 2^20 and the fractional part are exact in float32.
// (Equal, for every float32 in [0, 1], to shifting the mantissa by the
// exponent; checked exhaustively on the device.)
__device__ inline unsigned long long fixed_weight(float w) {
  const float a = w * 1048576.0f;
  const uint32_t hi = static_cast<uint32_t>(a);
  const uint32_t lo = static_cast<uint32_t>((a - static_cast<float>(hi)) * 1048576.0f);
  return (static_cast<unsigned long long>(hi) << 20) + lo;
}

// Processed probability of one entry of a row with statistics s.
__device__ inline float proc_prob(float z, const ProcStats &s, Temper invT) {
  if (!(s.mass > 0.0) || f32_order_key(z) < s.theta) return 0.0f;
  return proc_weight(z, s.zmax, invT) * s.inv_mass;
}

}  // namespace specv
