// Device and host helpers shared by the verify-and-commit kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "spec_verify.h"

namespace specv {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------- host ----
inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

// -------------------------------------------------------------- device ----
// Relaxed agent-scope (whole-GPU) atomic load: reads through the per-XCD L2s.
template <typename T>
__device__ inline T load_agent(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0 is folded onto +0 so the two compare equal, as they do as floats.
__device__ inline uint32_t f32_order_key(float v) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit argmax key: value order in the high word, (UINT32_MAX - index) in the
// low word, so the maximum key is the maximum value at the lowest index.
// Key 0 is below every real key and marks "no element".
__device__ inline uint64_t argmax_key(float v, int idx) {
  return (static_cast<uint64_t>(f32_order_key(v)) << 32) |
         static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(idx));
}
__device__ inline int argmax_key_index(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// DPP lane-move controls (CDNA): quad_perm [1,0,3,2] and [2,3,0,1] (lane xor 1
// and xor 2), and the mirrors within half rows (8 lanes) and rows (16 lanes).
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
// row_shr:n (n = 1, 2, 4, 8): lane i of a row of 16 reads lane i - n of the
// same row; the first n lanes of each row keep the `old` operand.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

// One DPP lane move of a 32- or 64-bit value (64-bit values move as two
// halves); lanes without a source take `old`.  Every lane of the wave must be
// active.
template <int CTRL, typename T>
__device__ inline T dpp_move(T v, T old) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                             CTRL, 0xF, 0xF, false));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v), o = __builtin_bit_cast(uint64_t, old);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(static_cast<uint32_t>(o)), static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(o >> 32), static_cast<int>(u >> 32), CTRL, 0xF, 0xF, false));
    return __builtin_bit_cast(T, (static_cast<uint64_t>(hi) << 32) | lo);
  }
}

// The value of lane `l` (uniform) of a 32- or 64-bit value.
template <typename T>
__device__ inline T read_lane(T v, int l) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), l));
    return __builtin_bit_cast(T, (static_cast<uint64_t>(hi) << 32) | lo);
  }
}

// Wave reduction by a commutative, associative op through DPP: butterflies
// inside each row of 16 lanes (xor 1, xor 2, half-row mirror, row mirror),
// then the four row results read as scalars.  Every lane of the wave must be
// active; every lane returns the result.
template <typename T, class Op>
__device__ inline T wave_reduce(T v, Op op) {
  v = op(v, dpp_move<kDppQuadXor1>(v, v));
  v = op(v, dpp_move<kDppQuadXor2>(v, v));
  v = op(v, dpp_move<kDppRowHalfMirror>(v, v));
  v = op(v, dpp_move<kDppRowMirror>(v, v));
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}

// Wave maximum through DPP lane moves (no LDS round trips): butterflies inside
// each row of 16 lanes (xor 1, xor 2, half-row mirror, row mirror leave every
// lane with its row's maximum), then the four row maxima are read as scalars.
// Every lane returns the wave maximum.
__device__ inline float wave_max_dpp(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, kDppQuadXor1, 0xF, 0xF, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, kDppQuadXor2, 0xF, 0xF, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, kDppRowHalfMirror, 0xF, 0xF, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, kDppRowMirror, 0xF, 0xF, false))));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(x, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(x, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(x, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(x, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ inline int wave_min(int v) {
  return wave_reduce(v, [](int a, int b) { return min(a, b); });
}
__device__ inline int wave_max_i(int v) {
  return wave_reduce(v, [](int a, int b) { return max(a, b); });
}
__device__ inline double wave_sum_d(double v) {
  return wave_reduce(v, [](double a, double b) { return a + b; });
}

// Inclusive scan across one wavefront (lane order); every lane of the wave
// must be active.  DPP row shifts give each row of 16 its own prefix, then the
// rows' totals (lanes 15, 31, 47) are added to the rows above.  For floating
// point this is a fixed order of additions (the same in every call).
template <typename T>
__device__ inline T wave_incl_scan(T v) {
  const int lane = threadIdx.x & (kWave - 1);
  v += dpp_move<kDppRowShr1>(v, T(0));
  v += dpp_move<kDppRowShr2>(v, T(0));
  v += dpp_move<kDppRowShr4>(v, T(0));
  v += dpp_move<kDppRowShr8>(v, T(0));
  const T r0 = read_lane(v, 15), r1 = read_lane(v, 31), r2 = read_lane(v, 47);
  const int row = lane >> 4;
  if (row >= 1) v += r0;
  if (row >= 2) v += r1;
  if (row >= 3) v += r2;
  return v;
}

// Block-wide exclusive sum of one int per thread (blockDim.x <= 1024).
// `sh` must hold blockDim.x / 64 ints.  Returns the exclusive prefix; *total
// receives the block total.  Contains barriers: call from every thread.
__device__ inline int block_excl_scan(int v, int *sh, int *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  int inc = wave_incl_scan(v);
  if (lane == kWave - 1) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    int x = lane < nw ? sh[lane] : 0;
    int xi = wave_incl_scan(x);
    if (lane < nw) sh[lane] = xi - x;
    if (lane == nw - 1) sh[nw] = xi;
  }
  __syncthreads();
  int r = inc - v + sh[w];
  *total = sh[nw];
  __syncthreads();
  return r;
}

// Exclusive prefix sum of n ints read with agent-scope loads, written to
// out[0..n], out[n] = total.  One block; contains barriers.
__device__ inline void block_offsets(const int32_t *in, int32_t *out, int n, int *sh) {
  const int T = blockDim.x;
  const int per = (n + T - 1) / T;
  const int lo = min(n, threadIdx.x * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += load_agent(in + i);
  int total;
  int base = block_excl_scan(s, sh, &total);
  for (int i = lo; i < hi; ++i) {
    out[i] = base;
    base += load_agent(in + i);
  }
  if (threadIdx.x == 0) out[n] = total;
}

}  // namespace specv
