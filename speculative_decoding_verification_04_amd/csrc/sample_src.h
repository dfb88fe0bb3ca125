// Row sources and the acceptance chain shared by the stochastic verification
// kernels (given float32 rows, or logits plus processed-row statistics).
//
// The rule is the Atlas lesson "Speculative decoding: proposals and verified
// output" (Acceptance and rejection correction) and the zero-to-sglang
// walkthrough 5.1: draft x_j is accepted when u_j < min(1, p_j(x_j) / q_j(x_j)),
// the first rejection stops the chain.
#pragma once

#include "process.h"

namespace specv {

struct SampleParams {
  const float *p, *q;           // dense rows (spec_verify_sample)
  const void *zp, *zq;          // logits (spec_verify_sample_logits)
  const ProcStats *sp, *sq;     // statistics of the processed rows
  Temper invT;                  // 1 / temperature
  const int32_t *draft;
  const float *u;
  int B, k, V, chunks;
  int vec;                      // rows are 16-byte aligned (V % 4 == 0 and aligned bases)
  int32_t eos;
  const int32_t *remaining;
  int32_t *accept_len, *emit_count, *out_tokens, *emit_offsets;
  double *final_mass;
  int32_t *status;
  unsigned long long *keys;     // [B * chunks] published chunk masses (0: not yet written)
  int32_t *ecnt;                // [B] published emit_count + 1 (0: not yet written)
};

// Stochastic verification from logits through the slices' candidate lists
// (top-k up to 256, or top-p alone): the slice launches, then the statistics
// and the draw in one launch; returns false, launching nothing, otherwise.
// P as for the verification, with P.sp / P.sq the statistics rows; list_ws
// the slice lists' workspace, list_idx proc_list_idx_bytes(rows), row_pub
// [rows][3] words (any contents).
bool launch_sample_logits_lists(const SampleParams &P, bool bf16, int top_k, float top_p, ProcStats *stats,
                                void *list_ws, int32_t *list_idx, unsigned long long *row_pub, hipStream_t s);

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kU = 4;                               // float4 loads in flight per lane
constexpr int kChunk = kThreads * 4 * kU;           // elements per chunk
constexpr int kEPT = kChunk / kThreads;             // elements per lane in the in-chunk scan
constexpr int kMaxChunks = 1024;                    // V <= kMaxChunks * kChunk

constexpr int kMaxPolls = 1 << 22;      // about 4 s of polling: a bound every wait reaches
enum : int { MODE_NONE = 0, MODE_RESID = 1, MODE_ROW = 2 };



// The mass vector a drawn token comes from: r_v = max(a_v - b_v, 0) when
// `resid` is set, else r_v = a_v.  DenseRow reads given float32 rows;
// LogitRow<BF16> computes the processed rows p', q' from logits on the fly.
struct DenseRow {
  const float *a, *b;
  bool resid;
  __device__ inline float at(int v) const { return resid ? fmaxf(a[v] - b[v], 0.0f) : a[v]; }
  // The 16 values v0 .. v0 + 15 (0 past V); 16-byte loads when `vec` (16-byte
  // aligned rows, v0 a multiple of 4) and the run is inside the row.
  __device__ inline void load16(float (&x)[16], int v0, int V, bool vec) const {
    if (vec && v0 + 16 <= V) {
      float4 A[4], Bv[4];
      const float4 *pa = reinterpret_cast<const float4 *>(a + v0);
#pragma unroll
      for (int u = 0; u < 4; ++u) A[u] = pa[u];
      if (resid) {
        const float4 *pb = reinterpret_cast<const float4 *>(b + v0);
#pragma unroll
        for (int u = 0; u < 4; ++u) Bv[u] = pb[u];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[4 * u + 0] = fmaxf(A[u].x - Bv[u].x, 0.0f);
          x[4 * u + 1] = fmaxf(A[u].y - Bv[u].y, 0.0f);
          x[4 * u + 2] = fmaxf(A[u].z - Bv[u].z, 0.0f);
          x[4 * u + 3] = fmaxf(A[u].w - Bv[u].w, 0.0f);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[4 * u + 0] = A[u].x;
          x[4 * u + 1] = A[u].y;
          x[4 * u + 2] = A[u].z;
          x[4 * u + 3] = A[u].w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = v0 + i < V ? at(v0 + i) : 0.0f;
    }
  }
};

template <bool BF16>
struct LogitRow {
  const void *a, *b;
  ProcStats sa, sb;
  Temper invT;
  bool resid;
  __device__ inline float at(int v) const {
    const float pa = proc_prob(logit_at<BF16>(a, v), sa, invT);
    return resid ? fmaxf(pa - proc_prob(logit_at<BF16>(b, v), sb, invT), 0.0f) : pa;
  }
  // 16 logits from v0 (a multiple of 8 for bf16, 4 for f32) as float32.
  __device__ static inline void load_z(float (&z)[16], const void *row, int v0) {
    if constexpr (BF16) {
      const uint4 *pr = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(row) + v0);
      const uint4 w0 = pr[0], w1 = pr[1];
      const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        z[2 * i] = __uint_as_float(w[i] << 16);
        z[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const float4 *pr = reinterpret_cast<const float4 *>(static_cast<const float *>(row) + v0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 f = pr[u];
        z[4 * u + 0] = f.x;
        z[4 * u + 1] = f.y;
        z[4 * u + 2] = f.z;
        z[4 * u + 3] = f.w;
      }
    }
  }
  // The 16 processed values v0 .. v0 + 15 (0 past V); 16-byte loads when
  // `vec` (16-byte aligned rows) and the run is inside the row.
  __device__ inline void load16(float (&x)[16], int v0, int V, bool vec) const {
    if (vec && v0 + 16 <= V) {
      float za[16], zb[16];
      load_z(za, a, v0);
      if (resid) load_z(zb, b, v0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pa = proc_prob(za[i], sa, invT);
        x[i] = resid ? fmaxf(pa - proc_prob(zb[i], sb, invT), 0.0f) : pa;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = v0 + i < V ? at(v0 + i) : 0.0f;
    }
  }
};

struct DenseSrc {
  using RowT = DenseRow;
  __device__ static inline float p_at(const SampleParams &P, int b, int j, int x) {
    return P.p[(static_cast<size_t>(b) * (P.k + 1) + j) * P.V + x];
  }
  __device__ static inline float q_at(const SampleParams &P, int b, int j, int x) {
    return P.q[(static_cast<size_t>(b) * P.k + j) * P.V + x];
  }
  __device__ static inline DenseRow row(const SampleParams &P, int b, int j, bool resid) {
    DenseRow r;
    r.a = P.p + (static_cast<size_t>(b) * (P.k + 1) + j) * P.V;
    r.b = resid ? P.q + (static_cast<size_t>(b) * P.k + j) * P.V : nullptr;
    r.resid = resid;
    return r;
  }
};

template <bool BF16>
struct LogitSrc {
  using RowT = LogitRow<BF16>;
  static constexpr size_t kElt = BF16 ? 2 : 4;
  __device__ static inline const void *prow(const SampleParams &P, int b, int j) {
    return static_cast<const unsigned char *>(P.zp) + (static_cast<size_t>(b) * (P.k + 1) + j) * P.V * kElt;
  }
  __device__ static inline const void *qrow(const SampleParams &P, int b, int j) {
    return static_cast<const unsigned char *>(P.zq) + (static_cast<size_t>(b) * P.k + j) * P.V * kElt;
  }
  __device__ static inline float p_at(const SampleParams &P, int b, int j, int x) {
    return proc_prob(logit_at<BF16>(prow(P, b, j), x), P.sp[static_cast<size_t>(b) * (P.k + 1) + j], P.invT);
  }
  __device__ static inline float q_at(const SampleParams &P, int b, int j, int x) {
    return proc_prob(logit_at<BF16>(qrow(P, b, j), x), P.sq[static_cast<size_t>(b) * P.k + j], P.invT);
  }
  __device__ static inline LogitRow<BF16> row(const SampleParams &P, int b, int j, bool resid) {
    LogitRow<BF16> r;
    r.a = prow(P, b, j);
    r.sa = P.sp[static_cast<size_t>(b) * (P.k + 1) + j];
    r.b = resid ? qrow(P, b, j) : nullptr;
    if (resid) r.sb = P.sq[static_cast<size_t>(b) * P.k + j];
    r.invT = P.invT;
    r.resid = resid;
    return r;
  }
};

template <typename T>
__device__ inline bool finite_val(T x) { return isfinite(x); }

// One draft's try: a = min(1, p(x) / q(x)) as one float32 division (q(x) = 0
// gives 1 when p(x) > 0, else 0); accepted iff u < a.  Returns the decision
// and its status bits.
__device__ inline int2 try_draft(float px, float qx, float u) {
  int st = 0;
  if (!finite_val(px) || !finite_val(qx)) st |= SPEC_ST_NONFINITE;
  float a;
  if (qx == 0.0f) {
    a = px > 0.0f ? 1.0f : 0.0f;
    st |= SPEC_ST_Q_ZERO;
  } else {
    const float ratio = __fdiv_rn(px, qx);
    a = ratio < 1.0f ? ratio : 1.0f;
  }
  return make_int2(u < a, st);
}

// The chain from the k tries in order (acc[j], st[j], the drafts d[j]): the
// first rejection stops it and the token is drawn from the residual of that
// row; after k acceptances the bonus comes from row k; EOS among the accepted
// drafts, or the budget rem (negative: none), ends the round without a draw.
// Returns x.mode, y.row drawn from, z.accepted drafts, w.status bits.
__device__ inline int4 fold_chain(int k, int rem, int eos, const int *acc, const int *sts, const int *d) {
  int mode = MODE_ROW, row = k, m = 0, st = 0;
  if (rem == 0) {
    mode = MODE_NONE;
  } else {
    for (int j = 0; j < k; ++j) {
      st |= sts[j];
      if (acc[j]) {
        ++m;
        if ((eos >= 0 && d[j] == eos) || m == rem) {
          mode = MODE_NONE;
          break;
        }
      } else {
        mode = MODE_RESID;
        row = j;
        break;
      }
    }
  }
  return make_int4(mode, row, m, st);
}

// The acceptance chain of sequence b, derived by every workgroup that needs
// it from the same gathers and the same float32 arithmetic (so all of them
// agree): x.mode, y.row drawn from, z.accepted drafts, w.status bits.
// Contains barriers.
template <class Src>
__device__ inline int4 derive_chain(const SampleParams &P, int b, int *sh_acc, int *sh_st, int *sh_d,
                                    int4 *sh_ch) {
  const int t = threadIdx.x;
  const int k = P.k, kp1 = k + 1, V = P.V;
  const int32_t *d = P.draft + static_cast<size_t>(b) * k;
  const float *ub = P.u + static_cast<size_t>(b) * kp1;
  const int rem = P.remaining ? P.remaining[b] : -1;   // negative: no budget (loaded with the drafts)
  for (int j = t; j < k; j += kThreads) {
    const int x = d[j];
    sh_d[j] = x;
    int2 r = make_int2(0, SPEC_ST_DRAFT_OOR);
    if (x >= 0 && x < V) r = try_draft(Src::p_at(P, b, j, x), Src::q_at(P, b, j, x), ub[j]);
    sh_acc[j] = r.x;
    sh_st[j] = r.y;
  }
  __syncthreads();
  if (t == 0) *sh_ch = fold_chain(k, rem, P.eos, sh_acc, sh_st, sh_d);
  __syncthreads();
  return *sh_ch;
}

// Emit offsets: the finishers publish emit_count + 1 per sequence as soon as
// their chains are known; one workgroup (any size up to 1024 lanes) scans
// them and clears the slots.
__device__ inline void finish_offsets(const SampleParams &P) {
  __shared__ int sh[1024 / kWave + 1];
  const int n = P.B, T = static_cast<int>(blockDim.x);
  const int per = (n + T - 1) / T;
  const int lo = min(n, static_cast<int>(threadIdx.x) * per), hi = min(n, lo + per);
  int polls = 0;
  while (true) {
    bool present = true;
    for (int i = lo; i < hi; ++i) present = present && load_agent(P.ecnt + i) != 0;
    if (__syncthreads_and(present)) break;
    if (++polls >= kMaxPolls) break;              // outputs unspecified; the wait still ends
    __builtin_amdgcn_s_sleep(1);
  }
  int s = 0;
  for (int i = lo; i < hi; ++i) s += max(load_agent(P.ecnt + i) - 1, 0);
  int total;
  int base = block_excl_scan(s, sh, &total);
  for (int i = lo; i < hi; ++i) {
    P.emit_offsets[i] = base;
    base += max(load_agent(P.ecnt + i) - 1, 0);
    P.ecnt[i] = 0;
  }
  if (threadIdx.x == 0) P.emit_offsets[n] = total;
}

}  // namespace
}  // namespace specv
