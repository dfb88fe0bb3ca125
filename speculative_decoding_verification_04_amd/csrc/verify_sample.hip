// Stochastic (Leviathan-style) verification of a batch of speculative rounds
// (gfx950).
//
// What it computes follows the Atlas lesson "Speculative decoding: proposals
// and verified output" (The mechanism, steps 2-5; Acceptance and rejection
// correction: a(x) = min(1, p(x)/q(x)), residual r = [p - q]_+ normalised)
// and the zero-to-sglang walkthrough 5.1 (accept when a uniform draw is below
// a; at a rejection draw the correction from the positive residual; bonus from
// the target after full acceptance).
//
// Design.  The acceptance chain only gathers 2 scalars per draft.  The bytes
// are in the single full row each sequence draws from: the residual
// p_j - q_j at the first rejection (8 bytes per vocabulary entry) or the
// target row p_k after full acceptance (4 bytes).  One launch:
//   * Producers, one workgroup per (sequence, chunk): each re-derives the
//     chain from the gathers, streams its chunk of the row with 16-byte loads
//     and publishes the chunk's float64 mass as a nonzero 64-bit key with an
//     agent-scope store.
//   * Finishers, one workgroup per sequence, after every producer in the
//     grid (workgroups are dispatched in index order, so a finisher is only
//     dispatched once every producer it waits on has been): each derives the
//     chain, writes the counts, polls its row's keys until all are present
//     (bounded), adds the masses in chunk order (S), finds the chunk whose
//     running sum first exceeds u * S, scans that chunk in index order and
//     writes the token; then it clears its keys, so the workspace is
//     zero-filled again for the next call.
//   * One last workgroup turns the emit counts (published by the finishers as
//     soon as their chains are known) into offsets.
// All sums are float64 over the float32 r_v in a fixed order, so results are
// reproducible run to run and within ~1e-16 relative of a correctly rounded
// sum.
#include "process.h"

namespace specv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kU = 4;                               // float4 loads in flight per lane
constexpr int kChunk = kThreads * 4 * kU;           // elements per chunk
constexpr int kEPT = kChunk / kThreads;             // elements per lane in the in-chunk scan
constexpr int kMaxChunks = 1024;                    // V <= kMaxChunks * kChunk

enum : int { MODE_NONE = 0, MODE_RESID = 1, MODE_ROW = 2 };

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

// Workspace: the chunk-mass slots, then the emit-count slots; zero-filled on
// entry and left zero-filled by every call.
struct SampleWs {
  size_t keys, ecnt, total;
};
inline SampleWs sample_ws_layout(int B, int chunks) {
  SampleWs w;
  w.keys = 0;
  w.ecnt = round_up(static_cast<size_t>(B) * chunks * sizeof(unsigned long long), 256);
  w.total = w.ecnt + round_up(static_cast<size_t>(B) * sizeof(int32_t), 256);
  return w;
}

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

__device__ inline double block_sum_d(double v, double *sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_sum_d(v);
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += sh[i];
  __syncthreads();
  return s;
}

// Block-wide exclusive sum of one double per lane, in a fixed order (lane
// order within a wave, then waves).  `sh` holds kWaves + 1 doubles; *total
// receives the block total.  Contains barriers.
__device__ inline double block_excl_scan_d(double v, double *sh, double *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const double inc = wave_incl_scan(v);
  if (lane == kWave - 1) sh[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) base += sh[i];
    tot += sh[i];
  }
  __syncthreads();
  *total = tot;
  return base + (inc - v);
}

static_assert(kEPT == 16, "a lane owns 16 consecutive entries of a chunk");

// Mass of chunk c of the row: lane t sums its 16 consecutive entries in order,
// then the lanes are added in a fixed tree.  Contains barriers.
template <class RowT>
__device__ inline double chunk_mass(const RowT &r, int c, int V, bool vec, double *sh) {
  float x[kEPT];
  r.load16(x, c * kChunk + threadIdx.x * kEPT, V, vec);
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kEPT; ++i) acc += static_cast<double>(x[i]);
  return block_sum_d(acc, sh);
}

template <typename T>
__device__ inline bool finite_val(T x) { return isfinite(x); }

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
    int st = 0, acc = 0;
    if (x >= 0 && x < V) {
      const float px = Src::p_at(P, b, j, x);
      const float qx = Src::q_at(P, b, j, x);
      if (!finite_val(px) || !finite_val(qx)) st |= SPEC_ST_NONFINITE;
      float a;
      if (qx == 0.0f) {
        a = px > 0.0f ? 1.0f : 0.0f;
        st |= SPEC_ST_Q_ZERO;
      } else {
        const float ratio = __fdiv_rn(px, qx);
        a = ratio < 1.0f ? ratio : 1.0f;
      }
      acc = ub[j] < a;
    } else {
      st |= SPEC_ST_DRAFT_OOR;
    }
    sh_acc[j] = acc;
    sh_st[j] = st;
  }
  __syncthreads();
  if (t == 0) {
    int mode = MODE_ROW, row = k, m = 0, st = 0;
    if (rem == 0) {
      mode = MODE_NONE;
    } else {
      for (int j = 0; j < k; ++j) {
        st |= sh_st[j];
        if (sh_acc[j]) {
          ++m;
          if ((P.eos >= 0 && sh_d[j] == P.eos) || m == rem) {
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
    *sh_ch = make_int4(mode, row, m, st);
  }
  __syncthreads();
  return *sh_ch;
}

// Chunk masses travel as 64-bit keys: the mass's bits XOR kMassSentinel.
// The sentinel is a NaN whose low 29 bits are not all zero, a pattern no mass
// here can take (a float32 widened to float64, and any arithmetic on such
// values, gives NaNs with those bits zero), so every published key is nonzero
// and a zero slot means "not yet written".
constexpr unsigned long long kMassSentinel = 0x7FF4000000000001ull;
constexpr int kMaxPolls = 1 << 22;      // about 4 s of polling: a bound every wait reaches

// Producer: chunk c of the row sequence b draws from; its mass published.
template <class Src>
__device__ inline void produce_chunk(const SampleParams &P, int b, int c) {
  __shared__ int sh_acc[SPEC_MAX_K], sh_st[SPEC_MAX_K], sh_d[SPEC_MAX_K];
  __shared__ int4 sh_ch;
  __shared__ double sh_red[kWaves];
  const int4 ch = derive_chain<Src>(P, b, sh_acc, sh_st, sh_d, &sh_ch);
  if (ch.x == MODE_NONE) return;                 // no draw: the finisher expects no mass
  const typename Src::RowT r = Src::row(P, b, ch.y, ch.x == MODE_RESID);
  const double part = chunk_mass(r, c, P.V, P.vec != 0, sh_red);
  if (threadIdx.x == 0)
    __hip_atomic_store(P.keys + static_cast<size_t>(b) * P.chunks + c,
                       static_cast<unsigned long long>(__double_as_longlong(part)) ^ kMassSentinel,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Finisher of sequence b: the chain's outputs, then (when a token is drawn)
// the chunk masses as they arrive, the draw, and every slot back to zero.
template <class Src>
__device__ inline void finish_sequence(const SampleParams &P, int b) {
  __shared__ int sh_acc[SPEC_MAX_K], sh_st[SPEC_MAX_K], sh_d[SPEC_MAX_K];
  __shared__ int4 sh_ch;
  __shared__ double sh_red[kWaves];
  __shared__ double sh_part[kMaxChunks];
  __shared__ int sh_scan[kWaves + 1];
  __shared__ int sh_last[kWaves];
  __shared__ double sh_dscan[kWaves + 1];
  __shared__ int sh_cs, sh_tok;
  __shared__ double sh_base;

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), w = t / kWave;
  const int k = P.k, kp1 = k + 1, V = P.V;
  const int nc = P.chunks;
  // loads that do not depend on the chain are issued with it
  const float u_draw = P.u[static_cast<size_t>(b) * kp1 + k];
  const int d_t = t < k ? P.draft[static_cast<size_t>(b) * k + t] : -1;
  const int4 ch = derive_chain<Src>(P, b, sh_acc, sh_st, sh_d, &sh_ch);
  const int mode = ch.x, jrow = ch.y, m = ch.z;
  const int emit = m + (mode != MODE_NONE ? 1 : 0);
  if (t == 0) {
    P.accept_len[b] = m;
    P.emit_count[b] = emit;
    if (P.emit_offsets) __hip_atomic_store(P.ecnt + b, emit + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  int st = ch.w;
  int tok = -1;
  double S = 0.0;
  if (mode != MODE_NONE) {
    unsigned long long *keys = P.keys + static_cast<size_t>(b) * nc;
    // wait until every chunk mass of the row is published (re-reading only
    // the missing ones); the bound keeps the wait finite
    int polls = 0;
    bool timed_out = false;
    while (true) {
      bool present = true;
      for (int i = t; i < nc; i += kThreads) {
        const unsigned long long key = load_agent(keys + i);
        if (key == 0ull) present = false;
        else sh_part[i] = __longlong_as_double(static_cast<long long>(key ^ kMassSentinel));
      }
      if (__syncthreads_and(present)) break;
      if (++polls >= kMaxPolls) {
        timed_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    for (int i = t; i < nc; i += kThreads) keys[i] = 0ull;   // ordered before the next call by the launch
    if (timed_out) {
      st |= SPEC_ST_INCOMPLETE;
    } else {
      typename Src::RowT r = Src::row(P, b, jrow, mode == MODE_RESID);
      const bool vec = P.vec != 0;
      const int per = (nc + kThreads - 1) / kThreads;  // chunks per lane, consecutive
      const int c0 = t * per;
      // total mass and each lane's exclusive prefix over the chunk masses
      double pre = 0.0;
      auto scan_parts = [&]() {
        double mine = 0.0;
        for (int i = 0; i < per; ++i)
          if (c0 + i < nc) mine += sh_part[c0 + i];
        pre = block_excl_scan_d(mine, sh_dscan, &S);
      };
      scan_parts();
      if (isfinite(S) && !(S > 0.0)) {
        st |= SPEC_ST_RESID_ZERO;
        if (mode == MODE_RESID) {         // fall back to the target row p_j itself
          r.resid = false;
          for (int i = 0; i < nc; ++i) {
            const double part = chunk_mass(r, i, V, vec, sh_red);
            if (t == 0) sh_part[i] = part;
          }
          __syncthreads();
          scan_parts();
        }
      }
      if (!isfinite(S)) {
        st |= SPEC_ST_NONFINITE;
        tok = 0;
      } else if (!(S > 0.0)) {
        tok = 0;
      } else {
        const double T = static_cast<double>(u_draw) * S;
        // the first chunk whose running mass exceeds T (else the last chunk with mass)
        int cand = INT_MAX, last = -1;
        {
          double run = pre;
          for (int i = 0; i < per; ++i) {
            const int c = c0 + i;
            if (c >= nc) break;
            const double pc = sh_part[c];
            if (pc > 0.0) last = c;
            if (cand == INT_MAX && run + pc > T) cand = c;
            run += pc;
          }
        }
        const int wc = wave_min(cand), wl = wave_max_i(last);
        if (lane == 0) {
          sh_scan[w] = wc;
          sh_last[w] = wl;
        }
        __syncthreads();
        if (t == 0) {
          int best = INT_MAX, lp = -1;
          for (int i = 0; i < kWaves; ++i) {
            best = min(best, sh_scan[i]);
            lp = max(lp, sh_last[i]);
          }
          sh_cs = best != INT_MAX ? best : lp;
        }
        __syncthreads();
        const int cs = sh_cs;
        if (cs >= c0 && cs < c0 + per) {                // the lane owning chunk cs: mass before it
          double run = pre;
          for (int c = c0; c < cs; ++c) run += sh_part[c];
          sh_base = run;
        }
        __syncthreads();
        const double base = sh_base;
        // in-chunk scan in index order: lane t owns kEPT consecutive entries
        const int lo = cs * kChunk + t * kEPT;
        float x[kEPT];
        r.load16(x, lo, V, vec);
        double mine = 0.0;
#pragma unroll
        for (int i = 0; i < kEPT; ++i) mine += static_cast<double>(x[i]);
        double ctot;
        double run = base + block_excl_scan_d(mine, sh_dscan, &ctot);
        int cpos = INT_MAX, lastpos = -1;
#pragma unroll
        for (int i = 0; i < kEPT; ++i) {
          const int v = lo + i;
          if (v < V) {
            if (x[i] > 0.0f) lastpos = v;
            run += static_cast<double>(x[i]);
            if (cpos == INT_MAX && run > T) cpos = v;
          }
        }
        const int wcp = wave_min(cpos), wlp = wave_max_i(lastpos);
        if (lane == 0) {
          sh_scan[w] = wcp;
          sh_last[w] = wlp;
        }
        __syncthreads();
        if (t == 0) {
          int best = INT_MAX, lp = -1;
          for (int i = 0; i < kWaves; ++i) {
            best = min(best, sh_scan[i]);
            lp = max(lp, sh_last[i]);
          }
          sh_tok = best != INT_MAX ? best : lp;
        }
        __syncthreads();
        tok = sh_tok;
      }
    }
  }
  if (t < kp1) {                                      // accepted drafts, then the drawn token
    int val = -1;
    if (t < m) val = d_t;
    else if (t == m && mode != MODE_NONE) val = tok;
    P.out_tokens[static_cast<size_t>(b) * kp1 + t] = val;
  }
  if (t == 0) {
    if (P.final_mass) P.final_mass[b] = mode != MODE_NONE ? S : 0.0;
    if (P.status) P.status[b] = st;
  }
}

// Emit offsets: the finishers publish emit_count + 1 per sequence as soon as
// their chains are known; one workgroup scans them and clears the slots.
__device__ inline void finish_offsets(const SampleParams &P) {
  __shared__ int sh[kWaves + 1];
  const int n = P.B, T = kThreads;
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

// One launch: B * chunks producers, then the B finishers, then (with
// offsets) the offsets workgroup.  Workgroups are dispatched in index order,
// so a waiting workgroup is dispatched only after every producer it waits on
// (producers never wait).
template <class Src>
__global__ __launch_bounds__(kThreads) void sample_verify_kernel(SampleParams P) {
  const int blk = blockIdx.x;
  const int nprod = P.B * P.chunks;
  if (blk < nprod) produce_chunk<Src>(P, blk / P.chunks, blk % P.chunks);
  else if (blk < nprod + P.B) finish_sequence<Src>(P, blk - nprod);
  else finish_offsets(P);
}

inline int sample_chunks(int V) { return (V + kChunk - 1) / kChunk; }

inline dim3 sample_grid(int B, int chunks, const void *emit_offsets) {
  return dim3(static_cast<unsigned>(static_cast<long long>(B) * chunks + B + (emit_offsets ? 1 : 0)));
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_sample_workspace_bytes(int B, int k, int V) {
  if (B < 1 || k < 1 || V < 1 || k > SPEC_MAX_K || sample_chunks(V) > kMaxChunks) return 0;
  return sample_ws_layout(B, sample_chunks(V)).total;
}

extern "C" int spec_verify_sample(const float *p, const float *q, const int32_t *draft,
                                  const float *uniforms, int B, int k, int V, int32_t eos_id,
                                  const int32_t *remaining, int32_t *accept_len,
                                  int32_t *emit_count, int32_t *out_tokens, int32_t *emit_offsets,
                                  double *final_mass, int32_t *status, void *ws, size_t ws_bytes,
                                  spec_stream_t stream) {
  if (!p || !q || !draft || !uniforms || !accept_len || !emit_count || !out_tokens || !ws)
    return SPEC_EINVAL;
  if (B < 1 || k < 1 || V < 1 || V >= INT32_MAX - 1) return SPEC_EINVAL;
  if (k > SPEC_MAX_K) return SPEC_ECAPACITY;
  const int chunks = sample_chunks(V);
  if (chunks > kMaxChunks) return SPEC_ECAPACITY;
  if (!aligned(p, 4) || !aligned(q, 4) || !aligned(uniforms, 4)) return SPEC_EINVAL;
  const long long nblocks = static_cast<long long>(B) * (chunks + 1) + 1;
  if (nblocks >= INT32_MAX) return SPEC_EINVAL;
  const SampleWs lay = sample_ws_layout(B, chunks);
  if (ws_bytes < lay.total || !aligned(ws, 256)) return SPEC_EWORKSPACE;

  const size_t np = static_cast<size_t>(B) * (k + 1) * V * 4, nq = static_cast<size_t>(B) * k * V * 4;
  const void *ins[] = {p, q, draft, uniforms, remaining, ws};
  const size_t in_n[] = {np, nq, static_cast<size_t>(B) * k * 4, static_cast<size_t>(B) * (k + 1) * 4,
                         static_cast<size_t>(B) * 4, lay.total};
  const void *outs[] = {accept_len, emit_count, out_tokens, emit_offsets, final_mass, status};
  const size_t out_n[] = {static_cast<size_t>(B) * 4, static_cast<size_t>(B) * 4,
                          static_cast<size_t>(B) * (k + 1) * 4, static_cast<size_t>(B + 1) * 4,
                          static_cast<size_t>(B) * 8, static_cast<size_t>(B) * 4};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }

  SampleParams P;
  P.p = p;
  P.q = q;
  P.zp = P.zq = nullptr;
  P.sp = P.sq = nullptr;
  P.invT = make_temper(1.0f);
  P.draft = draft;
  P.u = uniforms;
  P.B = B;
  P.k = k;
  P.V = V;
  P.chunks = chunks;
  P.vec = (V % 4 == 0) && aligned(p, 16) && aligned(q, 16);
  P.eos = eos_id;
  P.remaining = remaining;
  P.accept_len = accept_len;
  P.emit_count = emit_count;
  P.out_tokens = out_tokens;
  P.emit_offsets = emit_offsets;
  P.final_mass = final_mass;
  P.status = status;
  unsigned char *wb = static_cast<unsigned char *>(ws);
  P.keys = reinterpret_cast<unsigned long long *>(wb + lay.keys);
  P.ecnt = reinterpret_cast<int32_t *>(wb + lay.ecnt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(sample_verify_kernel<DenseSrc>, sample_grid(B, chunks, emit_offsets), dim3(kThreads), 0, s, P);
  return launch_status();
}

// Workspace of the verification from logits: per-row statistics of the
// B * (k+1) target and B * k draft rows, then the layout of spec_verify_sample.
static size_t sample_logits_stats_bytes(int B, int k, int V) {
  return round_up(static_cast<size_t>(B) * (2 * k + 1) * sizeof(ProcStats), 256) +
         proc_list_bytes(B * (2 * k + 1), V);
}

extern "C" size_t spec_verify_sample_logits_workspace_bytes(int B, int k, int V) {
  if (B < 1 || k < 1 || V < 1 || k > SPEC_MAX_K || V > SPEC_PROC_MAX_V || sample_chunks(V) > kMaxChunks) return 0;
  return sample_logits_stats_bytes(B, k, V) + sample_ws_layout(B, sample_chunks(V)).total;
}

extern "C" int spec_verify_sample_logits(const void *target_logits, const void *draft_logits,
                                         spec_dtype dt, int B, int k, int V, float temperature,
                                         int top_k, float top_p, const int32_t *draft,
                                         const float *uniforms, int32_t eos_id,
                                         const int32_t *remaining, int32_t *accept_len,
                                         int32_t *emit_count, int32_t *out_tokens,
                                         int32_t *emit_offsets, double *final_mass,
                                         int32_t *status, void *ws, size_t ws_bytes,
                                         spec_stream_t stream) {
  if (!target_logits || !draft_logits || !draft || !uniforms || !accept_len || !emit_count ||
      !out_tokens || !ws)
    return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (B < 1 || k < 1 || !proc_args_ok(temperature, top_k, top_p, V)) return SPEC_EINVAL;
  if (k > SPEC_MAX_K) return SPEC_ECAPACITY;
  const int chunks = sample_chunks(V);
  if (chunks > kMaxChunks) return SPEC_ECAPACITY;
  const size_t elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(target_logits, elt) || !aligned(draft_logits, elt) || !aligned(uniforms, 4)) return SPEC_EINVAL;
  const long long nblocks = static_cast<long long>(B) * (chunks + 1) + 1;
  const long long rows = static_cast<long long>(B) * (2 * k + 1);
  if (nblocks >= INT32_MAX || rows >= INT32_MAX) return SPEC_EINVAL;
  const size_t stats_bytes = sample_logits_stats_bytes(B, k, V);
  const SampleWs lay = sample_ws_layout(B, chunks);
  if (ws_bytes < stats_bytes + lay.total || !aligned(ws, 256)) return SPEC_EWORKSPACE;

  const size_t np = static_cast<size_t>(B) * (k + 1) * V * elt, nq = static_cast<size_t>(B) * k * V * elt;
  const void *ins[] = {target_logits, draft_logits, draft, uniforms, remaining, ws};
  const size_t in_n[] = {np, nq, static_cast<size_t>(B) * k * 4, static_cast<size_t>(B) * (k + 1) * 4,
                         static_cast<size_t>(B) * 4, stats_bytes + lay.total};
  const void *outs[] = {accept_len, emit_count, out_tokens, emit_offsets, final_mass, status};
  const size_t out_n[] = {static_cast<size_t>(B) * 4, static_cast<size_t>(B) * 4,
                          static_cast<size_t>(B) * (k + 1) * 4, static_cast<size_t>(B + 1) * 4,
                          static_cast<size_t>(B) * 8, static_cast<size_t>(B) * 4};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }

  unsigned char *wb = static_cast<unsigned char *>(ws);
  ProcStats *stats = reinterpret_cast<ProcStats *>(wb);
  SampleParams P;
  P.p = P.q = nullptr;
  P.zp = target_logits;
  P.zq = draft_logits;
  P.sp = stats;                                   // target rows first
  P.sq = stats + static_cast<size_t>(B) * (k + 1); // then the draft rows
  P.invT = make_temper(temperature);
  P.draft = draft;
  P.u = uniforms;
  P.B = B;
  P.k = k;
  P.V = V;
  P.chunks = chunks;
  P.vec = (V % (dt == SPEC_BF16 ? 8 : 4) == 0) && aligned(target_logits, 16) && aligned(draft_logits, 16);
  P.eos = eos_id;
  P.remaining = remaining;
  P.accept_len = accept_len;
  P.emit_count = emit_count;
  P.out_tokens = out_tokens;
  P.emit_offsets = emit_offsets;
  P.final_mass = final_mass;
  P.status = status;
  P.keys = reinterpret_cast<unsigned long long *>(wb + stats_bytes + lay.keys);
  P.ecnt = reinterpret_cast<int32_t *>(wb + stats_bytes + lay.ecnt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dt == SPEC_BF16;
  (void)hipGetLastError();
  launch_proc_stats(target_logits, draft_logits, B * (k + 1), static_cast<int>(rows), V, bf16, P.invT,
                    top_k, top_p, stats, nullptr,
                    wb + round_up(static_cast<size_t>(rows) * sizeof(ProcStats), 256), s);
  const dim3 grid = sample_grid(B, chunks, emit_offsets), blk(kThreads);
  if (bf16)
    hipLaunchKernelGGL(sample_verify_kernel<LogitSrc<true>>, grid, blk, 0, s, P);
  else
    hipLaunchKernelGGL(sample_verify_kernel<LogitSrc<false>>, grid, blk, 0, s, P);
  return launch_status();
}
