// Row statistics of processed sampling distributions (temperature, top-k,
// top-p) and their optional materialisation (gfx950).
//
// Definitions: process.h (after the zero-to-sglang walkthrough 5.1, which
// requires the processed probabilities to be the ones verified).
//
// Design.  One 1024-lane workgroup per row; the row is read once from HBM and
// then re-read from L2 by the later passes (a 151936-entry bf16 row is 297 KB,
// a few rows per XCD fit its 4 MB L2):
//   1. row maximum;
//   2. top-k: radix selection of the K-th largest order key, 8 bits per pass
//      (2 passes for bf16, whose keys carry 16 significant bits; 4 for f32),
//      with a 256-bin count histogram in LDS;
//   3. top-p: the same descent over the top-k survivors with a 256-bin
//      histogram of counts and of fixed-point weights (2^-44 units, integer
//      LDS atomics, so the selection is reproducible): at each level the
//      lowest bucket whose top value still has less than top_p of the total
//      weight above it holds the boundary value;
//   4. the kept weight as a float64 sum in a fixed order, and, if asked, p'
//      written for every entry.
// Every selection keeps all logits at or above one threshold, so ties at a
// boundary are kept, as the definitions require.
#include "process.h"

namespace specv {
namespace {

constexpr int kProcThreads = 1024;
constexpr int kProcWaves = kProcThreads / kWave;
constexpr int kProcU = 4;                      // 16-byte loads in flight per lane
constexpr double kFixScale = 17592186044416.0;  // 2^44 fixed-point units per unit weight

struct ProcParams {
  const void *za, *zb;   // rows [0, rows_a) come from za, the rest from zb
  int rows_a, rows, V;
  ProcConfig cfg;
  ProcStats *stats;      // [rows]
  float *probs;          // [rows, V] or null
};

template <bool BF16>
__device__ inline const void *proc_row(const ProcParams &P, int r) {
  const size_t elt = BF16 ? 2 : 4;
  if (r < P.rows_a) return static_cast<const unsigned char *>(P.za) + static_cast<size_t>(r) * P.V * elt;
  return static_cast<const unsigned char *>(P.zb) + static_cast<size_t>(r - P.rows_a) * P.V * elt;
}

// Calls f(v, z) for every entry of the row this lane owns: a scalar head up to
// the first 16-byte boundary, 16-byte vectors (kProcU in flight per lane),
// a scalar tail.  The order within a lane is fixed, so sums are reproducible.
template <bool BF16, class F>
__device__ inline void row_foreach(const void *row, int V, F &&f) {
  constexpr int ELT = BF16 ? 2 : 4, VEC = 16 / ELT;
  const int t = threadIdx.x;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row);
  const int head = min(V, static_cast<int>(((16u - (a & 15u)) & 15u) / ELT));
  const int nvec = (V - head) / VEC;
  const int tail0 = head + nvec * VEC;
  if (t < head) f(t, logit_at<BF16>(row, t));
  const uint4 *body = reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(row) + head * ELT);
  for (int i0 = 0; i0 < nvec; i0 += kProcThreads * kProcU) {
    uint4 x[kProcU];
#pragma unroll
    for (int u = 0; u < kProcU; ++u) {
      const int i = i0 + u * kProcThreads + t;
      if (i < nvec) x[u] = body[i];
    }
#pragma unroll
    for (int u = 0; u < kProcU; ++u) {
      const int i = i0 + u * kProcThreads + t;
      if (i < nvec) {
        const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
        const int v0 = head + i * VEC;
        if constexpr (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f(v0 + 2 * e, __uint_as_float(w[e] << 16));
            f(v0 + 2 * e + 1, __uint_as_float(w[e] & 0xFFFF0000u));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) f(v0 + e, __uint_as_float(w[e]));
        }
      }
    }
  }
  if (t < V - tail0) f(tail0 + t, logit_at<BF16>(row, tail0 + t));
}

__device__ inline float block_max_f(float v, float *sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_max_dpp(v);
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float m = sh[0];
#pragma unroll
  for (int i = 1; i < kProcWaves; ++i) m = fmaxf(m, sh[i]);
  __syncthreads();
  return m;
}

__device__ inline double block_sum_dd(double v, double *sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_sum_d(v);
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kProcWaves; ++i) s += sh[i];
  __syncthreads();
  return s;
}

template <bool BF16>
__global__ __launch_bounds__(kProcThreads) void proc_stats_kernel(ProcParams P) {
  __shared__ uint32_t h_cnt[256];
  __shared__ unsigned long long h_mass[256];
  __shared__ float sh_f[kProcWaves];
  __shared__ double sh_d[kProcWaves];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_need;
  __shared__ unsigned long long sh_above;
  __shared__ double sh_thr;

  const int t = threadIdx.x;
  const int r = blockIdx.x;
  const int V = P.V;
  const void *row = proc_row<BF16>(P, r);
  constexpr int kLevels = BF16 ? 2 : 4;        // 8-bit digits of the significant key bits
  const float T = P.cfg.T;

  // 1. row maximum
  float m = -INFINITY;
  row_foreach<BF16>(row, V, [&](int, float z) { m = fmaxf(m, z); });
  const float zmax = block_max_f(m, sh_f);

  // 2. top-k: the K-th largest key, one 8-bit digit per pass
  uint32_t tau = 0;
  const int K = P.cfg.top_k;
  if (K > 0 && K < V) {
    uint32_t prefix = 0, pmask = 0;
    int need = K;
    for (int lvl = 0; lvl < kLevels; ++lvl) {
      const int shift = 24 - 8 * lvl;
      for (int i = t; i < 256; i += kProcThreads) h_cnt[i] = 0;
      __syncthreads();
      row_foreach<BF16>(row, V, [&](int, float z) {
        const uint32_t key = f32_order_key(z);
        if ((key & pmask) == prefix) atomicAdd(&h_cnt[(key >> shift) & 255u], 1u);
      });
      __syncthreads();
      if (t == 0) {
        int above = 0, d = 255;
        for (; d > 0; --d) {
          if (above + static_cast<int>(h_cnt[d]) >= need) break;
          above += static_cast<int>(h_cnt[d]);
        }
        sh_need = need - above;
        sh_prefix = prefix | (static_cast<uint32_t>(d) << shift);
      }
      __syncthreads();
      need = sh_need;
      prefix = sh_prefix;
      pmask |= 255u << shift;
    }
    tau = prefix;   // the smallest key with the selected significant bits
  }

  // 3. top-p over the top-k survivors
  uint32_t theta = tau;
  if (P.cfg.top_p < 1.0f && zmax != -INFINITY) {
    uint32_t prefix = 0, pmask = 0;
    unsigned long long above = 0;
    bool found = true;
    for (int lvl = 0; lvl < kLevels; ++lvl) {
      const int shift = 24 - 8 * lvl;
      for (int i = t; i < 256; i += kProcThreads) {
        h_cnt[i] = 0;
        h_mass[i] = 0ull;
      }
      __syncthreads();
      row_foreach<BF16>(row, V, [&](int, float z) {
        const uint32_t key = f32_order_key(z);
        if (key >= tau && (key & pmask) == prefix) {
          const uint32_t d = (key >> shift) & 255u;
          atomicAdd(&h_cnt[d], 1u);
          const double wq = static_cast<double>(proc_weight(z, zmax, T)) * kFixScale;
          atomicAdd(&h_mass[d], static_cast<unsigned long long>(__double2ull_rn(wq)));
        }
      });
      __syncthreads();
      if (t == 0) {
        if (lvl == 0) {
          unsigned long long tot = 0;
          for (int d = 0; d < 256; ++d) tot += h_mass[d];
          sh_thr = static_cast<double>(P.cfg.top_p) * static_cast<double>(tot);
        }
        const double thr = sh_thr;
        unsigned long long run = above, astar = above;
        int dstar = -1;
        for (int d = 255; d >= 0; --d) {       // buckets from the largest logits down
          if (h_cnt[d] == 0) continue;
          if (static_cast<double>(run) < thr) {
            dstar = d;                           // this bucket's top value is kept
            astar = run;
          } else {
            break;
          }
          run += h_mass[d];
        }
        sh_prefix = dstar < 0 ? 0xFFFFFFFFu : (prefix | (static_cast<uint32_t>(dstar) << shift));
        sh_above = astar;
      }
      __syncthreads();
      if (sh_prefix == 0xFFFFFFFFu) {          // no weight at all: keep the top-k set
        found = false;
        break;
      }
      prefix = sh_prefix;
      above = sh_above;
      pmask |= 255u << shift;
    }
    if (found) theta = prefix;
  }

  // 4. kept weight (fixed order), smallest kept logit and, if asked, the
  //    processed row
  double acc = 0.0;
  float zlo = INFINITY;
  row_foreach<BF16>(row, V, [&](int, float z) {
    if (f32_order_key(z) >= theta) {
      acc += static_cast<double>(proc_weight(z, zmax, T));
      zlo = fminf(zlo, z);
    }
  });
  const double mass = block_sum_dd(acc, sh_d);
  const float zmin_kept = -block_max_f(-zlo, sh_f);
  ProcStats st;
  st.zmax = zmax;
  st.theta = theta;
  st.mass = mass;
  st.inv_mass = mass > 0.0 ? static_cast<float>(1.0 / mass) : 0.0f;
  st.zmin_kept = zmin_kept;
  if (t == 0) P.stats[r] = st;
  if (P.probs) {
    float *out = P.probs + static_cast<size_t>(r) * V;
    row_foreach<BF16>(row, V, [&](int v, float z) { out[v] = proc_prob(z, st, T); });
  }
}

__global__ __launch_bounds__(256) void proc_export_kernel(const ProcStats *stats, int R, float *row_max,
                                                          float *row_threshold, double *row_mass) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const ProcStats st = stats[r];
  if (row_max) row_max[r] = st.zmax;
  if (row_threshold) row_threshold[r] = st.zmin_kept;
  if (row_mass) row_mass[r] = st.mass;
}

}  // namespace

// Launches the statistics kernel over rows [0, rows); shared with the
// stochastic verification from logits.
int launch_proc_stats(const void *za, const void *zb, int rows_a, int rows, int V, bool bf16,
                      float T, int top_k, float top_p, ProcStats *stats, float *probs,
                      hipStream_t s) {
  ProcParams P;
  P.za = za;
  P.zb = zb;
  P.rows_a = rows_a;
  P.rows = rows;
  P.V = V;
  P.cfg.T = T;
  P.cfg.top_k = top_k;
  P.cfg.top_p = top_p;
  P.stats = stats;
  P.probs = probs;
  if (bf16)
    hipLaunchKernelGGL(proc_stats_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(kProcThreads), 0, s, P);
  else
    hipLaunchKernelGGL(proc_stats_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(kProcThreads), 0, s, P);
  return 0;
}

bool proc_args_ok(float T, int top_k, float top_p, int V) {
  return T > 0.0f && T < INFINITY && top_k >= 0 && top_p > 0.0f && top_p <= 1.0f &&
         V >= 1 && V <= SPEC_PROC_MAX_V;
}

}  // namespace specv

using namespace specv;

extern "C" size_t spec_process_workspace_bytes(int R) {
  if (R < 1) return 0;
  return round_up(static_cast<size_t>(R) * sizeof(ProcStats), 256);
}

extern "C" int spec_process_logits(const void *logits, spec_dtype dt, int R, int V, float temperature,
                                   int top_k, float top_p, float *probs, float *row_max,
                                   float *row_threshold, double *row_mass, void *ws, size_t ws_bytes,
                                   spec_stream_t stream) {
  if (!logits || !ws) return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (R < 1 || !proc_args_ok(temperature, top_k, top_p, V)) return SPEC_EINVAL;
  const size_t elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(logits, elt)) return SPEC_EINVAL;
  const size_t need = spec_process_workspace_bytes(R);
  if (ws_bytes < need || !aligned(ws, 256)) return SPEC_EWORKSPACE;
  const size_t nz = static_cast<size_t>(R) * V * elt;
  const void *ins[] = {logits, ws};
  const size_t in_n[] = {nz, need};
  void *outs[] = {probs, row_max, row_threshold, row_mass};
  const size_t out_n[] = {static_cast<size_t>(R) * V * 4, static_cast<size_t>(R) * 4,
                          static_cast<size_t>(R) * 4, static_cast<size_t>(R) * 8};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 2; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  ProcStats *stats = static_cast<ProcStats *>(ws);
  (void)hipGetLastError();
  launch_proc_stats(logits, logits, R, R, V, dt == SPEC_BF16, temperature, top_k, top_p, stats, probs, s);
  if (row_max || row_threshold || row_mass)
    hipLaunchKernelGGL(proc_export_kernel, dim3((R + 255) / 256), dim3(256), 0, s, stats, R, row_max,
                       row_threshold, row_mass);
  return launch_status();
}
