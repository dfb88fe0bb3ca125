// Stochastic verification of a candidate tree (gfx950).
//
// What it computes: the rule of the Atlas lesson "Speculative decoding:
// proposals and verified output" (Acceptance and rejection correction) and
// the zero-to-sglang walkthrough 5.1, applied along a tree whose siblings were
// drawn independently from the draft's distribution at their parent (the
// walkthrough 5.2 lists the draft tokens and their draft probabilities among
// a tree verifier's fields; the "Correctness Forensics" summary, section 5,
// names tree verification): the children of the current node are tried in
// sibling order against the current residual of the target row; after a
// rejection the residual becomes the normalised positive part of
// (residual - q); an accepted child becomes the current node; when no child
// is accepted, or at a leaf, one token is drawn from the current residual.
// A chain tree is exactly the linear stochastic verification.
//
// The residual after i rejections at a node is never stored: with R_0 = p,
// R_1 = max(p - q, 0) in float32 and R_j = max(R_{j-1} - q * m_{j-1}, 0) in
// float64 (m_j the sum of R_j), R_i(v) is recomputed from p(v), q(v) and the
// masses m_1 .. m_{i-1} kept in LDS.  Every step that the rounding of the
// result depends on is a separately rounded IEEE operation (no contraction).
//
// Design.  One workgroup of 1024 lanes per sequence walks its tree.  Lane 0
// decides each try from two gathers; a rejection runs one pass over the
// node's p and q rows (four chunks of 4096 entries per step, one per quarter
// of the workgroup, the next step's loads issued before this step's sums),
// giving the next residual's chunk masses (fixed-order float64 sums) in LDS;
// the draw scans those masses for the chunk that crosses u * S and then that
// chunk in index order, as the linear verification does.  Sequences are
// independent, so no workgroup waits for another; a second launch scans the
// emit counts into offsets.
#include "common.h"

namespace specv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kQuarter = 256;                      // lanes per chunk
constexpr int kEPT = 16;                           // entries per lane per chunk
constexpr int kChunk = kQuarter * kEPT;            // 4096 entries
constexpr int kChunksPerStep = kThreads / kQuarter;
constexpr int kMaxChunks = 1024;                   // V <= kMaxChunks * kChunk
constexpr int kMaxLevels = SPEC_TREE_MAX_N;        // rejections at one node <= its children < N

struct TreeSampleParams {
  const float *p, *q;            // [B, N, V]
  const int32_t *draft, *first_child, *next_sibling;   // [B, N]
  const float *u;                // [B, N]
  int B, N, V, chunks;
  int vec;                       // rows 16-byte aligned (V % 4 == 0 and aligned bases)
  int32_t eos;
  const int32_t *remaining;
  int32_t *accept_len, *emit_count, *out_tokens, *path, *emit_offsets;
  double *final_mass;
  int32_t *status;
  int W;                         // workgroups per sequence (1: one walks alone)
  unsigned long long *slots;     // [B][N][chunks] published chunk masses, per pass (W > 1)
  int32_t *done;                 // [B][W] members finished with the slots (W > 1)
};

// Chunk masses travel between the workgroups of a sequence as 64-bit keys: the
// mass's bits XOR kMassSentinel, a NaN whose low 29 bits are not all zero --
// a pattern no sum of float32 values widened to float64 takes -- so every
// published key is nonzero and a zero slot means "not yet written".
constexpr unsigned long long kMassSentinel = 0x7FF4000000000001ull;
constexpr int kMaxPolls = 1 << 22;               // about 4 s of polling: a bound every wait reaches
constexpr int kMaxCoopGroups = 128;              // B * W: one workgroup per CU, all resident at once
constexpr int kMaxMembers = 16;
constexpr long long kMaxCoopSlots = 8LL << 20;   // B * N * chunks: 64 MB of slots at most

// R_i(v) from p(v), q(v) and the masses m[1 .. i-1] (m[0] unused).  R_0 = p as
// given, R_1 = max(p - q, 0) in float32, then float64 steps.
__device__ inline double resid_at(float pv, float qv, int i, const double *m) {
#pragma clang fp contract(off)
  if (i == 0) return static_cast<double>(pv);
  double r = static_cast<double>(fmaxf(pv - qv, 0.0f));
  const double qd = static_cast<double>(qv);
  for (int j = 2; j <= i; ++j) {
    const double t = r - qd * m[j - 1];
    r = t > 0.0 ? t : 0.0;
  }
  return r;
}

// The acceptance test of a try after i >= 1 rejections: u < R_i(x) / (m_i q(x)).
__device__ inline bool accept_resid(double rx, double mi, float qx, float u, int *st) {
#pragma clang fp contract(off)
  if (!isfinite(rx) || !isfinite(qx)) *st |= SPEC_ST_NONFINITE;
  double a;
  if (qx == 0.0f) {
    a = rx > 0.0 ? 1.0 : 0.0;
    *st |= SPEC_ST_Q_ZERO;
  } else {
    const double den = mi * static_cast<double>(qx);
    a = rx / den;
    if (!(a < 1.0)) a = 1.0;
  }
  return static_cast<double>(u) < a;
}

// 16 consecutive entries of a row from v0 (0 past V): four 16-byte loads when
// the row is aligned and the run inside it.
__device__ inline void load16(float (&x)[kEPT], const float *row, int v0, int V, bool vec) {
  if (vec && v0 + kEPT <= V) {
    const float4 *pr = reinterpret_cast<const float4 *>(row + v0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 f = pr[u];
      x[4 * u + 0] = f.x;
      x[4 * u + 1] = f.y;
      x[4 * u + 2] = f.z;
      x[4 * u + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kEPT; ++i) x[i] = v0 + i < V ? row[v0 + i] : 0.0f;
  }
}

struct Shared {
  int fc[SPEC_TREE_MAX_N], ns[SPEC_TREE_MAX_N], d[SPEC_TREE_MAX_N];
  float u[SPEC_TREE_MAX_N];
  int out[SPEC_TREE_MAX_N], nodes[SPEC_TREE_MAX_N];
  double m[kMaxLevels + 1];               // masses of R_1 .. R_i at the current node
  double part[2][kMaxChunks];             // chunk masses: the current residual, the candidate
  double wsum[kWaves];
  double dscan[kWaves + 1];
  int iscan[kWaves], ilast[kWaves];
  int flag, tok, cs;
  double base;
};

__device__ inline unsigned long long mass_key(double m) {
  return static_cast<unsigned long long>(__double_as_longlong(m)) ^ kMassSentinel;
}

// Chunk masses of R_i over the row pair (p, q) into part[], and their total in
// chunk order.  Member w of the W workgroups of a sequence computes chunks
// w, w + W, w + 2W, ...: each quarter of the workgroup takes one of them per
// step (the next step's loads issued before this step's sums), a lane adds
// its 16 entries in index order and the quarter's four waves are added in
// order (the order of the linear verification's chunk masses).  With W > 1 the
// masses are published into this pass's slots and the member waits (bounded)
// for every other chunk's; *timed_out reports a wait that did not end.  The
// total adds the masses as the linear verification does: 256 lanes, each a run
// of consecutive chunks, then a fixed-order scan.  Contains barriers.
__device__ double residual_pass(const TreeSampleParams &P, const float *prow, const float *qrow, int i,
                                Shared &S, double *part, int w, unsigned long long *slots, bool *timed_out) {
  const int t = threadIdx.x, quarter = t / kQuarter, ql = t % kQuarter, lane = t & (kWave - 1);
  const int wv = t / kWave;
  const bool vec = P.vec != 0;
  const int W = P.W;
  const int nown = w < P.chunks ? (P.chunks - w + W - 1) / W : 0;   // this member's chunks
  const int steps = (nown + kChunksPerStep - 1) / kChunksPerStep;
  float xp[kEPT], xq[kEPT], np_[kEPT], nq[kEPT];
#pragma unroll
  for (int e = 0; e < kEPT; ++e) xp[e] = xq[e] = np_[e] = nq[e] = 0.0f;   // q is not read for R_0
  int j = quarter;                            // this quarter's own-chunk index
  if (steps > 0) {
    const int c = w + W * j;
    load16(xp, prow, c * kChunk + ql * kEPT, P.V, vec);
    if (i > 0) load16(xq, qrow, c * kChunk + ql * kEPT, P.V, vec);
  }
  for (int s = 0; s < steps; ++s) {
    const int jn = j + kChunksPerStep;
    if (s + 1 < steps) {                     // the next step's loads before this step's sums
      const int cn = w + W * jn;
      load16(np_, prow, cn * kChunk + ql * kEPT, P.V, vec);
      if (i > 0) load16(nq, qrow, cn * kChunk + ql * kEPT, P.V, vec);
    }
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) acc += resid_at(xp[e], xq[e], i, S.m);
    acc = wave_sum_d(acc);
    if (lane == 0) S.wsum[wv] = acc;
    __syncthreads();
    if (ql == 0 && j < nown) {
      const int c = w + W * j;
      const int w0 = quarter * (kQuarter / kWave);
      double tot = 0.0;
      for (int k = 0; k < kQuarter / kWave; ++k) tot += S.wsum[w0 + k];
      part[c] = tot;
      if (W > 1) __hip_atomic_store(slots + c, mass_key(tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    j = jn;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      xp[e] = np_[e];
      xq[e] = nq[e];
    }
  }
  if (W > 1) {                               // every other member's chunks
    int polls = 0;
    while (true) {
      bool present = true;
      for (int c = t; c < P.chunks; c += kThreads) {
        if (c % W == w) continue;
        const unsigned long long key = load_agent(slots + c);
        if (key == 0ull) present = false;
        else part[c] = __longlong_as_double(static_cast<long long>(key ^ kMassSentinel));
      }
      if (__syncthreads_and(present)) break;
      if (++polls >= kMaxPolls) {
        *timed_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  const int per = (P.chunks + kQuarter - 1) / kQuarter;
  double mine = 0.0;
  for (int k = 0; k < per; ++k) {
    const int cc = t * per + k;
    if (cc < P.chunks) mine += part[cc];
  }
  double inc = wave_incl_scan(mine);
  if (lane == kWave - 1) S.dscan[wv] = inc;
  __syncthreads();
  double tot = 0.0;
  for (int k = 0; k < kWaves; ++k) tot += S.dscan[k];
  __syncthreads();
  return tot;
}

// Block-wide exclusive sum of one double per lane in a fixed order (lane order
// within a wave, then waves); *total gets the sum.  Contains barriers.
__device__ inline double block_excl_scan_d(double v, Shared &S, double *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const double inc = wave_incl_scan(v);
  if (lane == kWave - 1) S.dscan[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) base += S.dscan[k];
    tot += S.dscan[k];
  }
  __syncthreads();
  *total = tot;
  return base + (inc - v);
}

// One draw with uniform u from R_i of the row pair, whose chunk masses are in
// part[] and total in Stot: the first chunk whose running mass exceeds u * S,
// then the first entry inside it (the last chunk or entry with mass when
// rounding leaves none).  Contains barriers.
__device__ int draw_token(const TreeSampleParams &P, const float *prow, const float *qrow, int i, Shared &S,
                          const double *part, double Stot, float u) {
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const double T = static_cast<double>(u) * Stot;
  const int nc = P.chunks;
  const int per = (nc + kQuarter - 1) / kQuarter;   // lanes 0 .. 255 hold the chunks, as in the linear draw
  const int c0 = t * per;
  double mine = 0.0;
  for (int k = 0; k < per; ++k)
    if (c0 + k < nc) mine += part[c0 + k];
  double dummy;
  const double pre = block_excl_scan_d(mine, S, &dummy);
  int cand = INT_MAX, last = -1;
  {
    double run = pre;
    for (int k = 0; k < per; ++k) {
      const int c = c0 + k;
      if (c >= nc) break;
      const double pc = part[c];
      if (pc > 0.0) last = c;
      if (cand == INT_MAX && run + pc > T) cand = c;
      run += pc;
    }
  }
  const int wc = wave_min(cand), wl = wave_max_i(last);
  if (lane == 0) {
    S.iscan[w] = wc;
    S.ilast[w] = wl;
  }
  __syncthreads();
  if (t == 0) {
    int best = INT_MAX, lp = -1;
    for (int k = 0; k < kWaves; ++k) {
      best = min(best, S.iscan[k]);
      lp = max(lp, S.ilast[k]);
    }
    S.cs = best != INT_MAX ? best : lp;
  }
  __syncthreads();
  const int cs = min(max(S.cs, 0), nc - 1);     // S > 0 and finite: some chunk has mass
  if (cs >= c0 && cs < c0 + per) {              // the lane owning chunk cs: mass before it
    double run = pre;
    for (int c = c0; c < cs; ++c) run += part[c];
    S.base = run;
  }
  __syncthreads();
  const double base = S.base;
  // in-chunk scan in index order: lanes 0 .. 255 own 16 consecutive entries
  float xp[kEPT], xq[kEPT];
#pragma unroll
  for (int e = 0; e < kEPT; ++e) xp[e] = xq[e] = 0.0f;
  const int lo = cs * kChunk + t * kEPT;
  const bool active = t < kQuarter;
  if (active) {
    load16(xp, prow, lo, P.V, P.vec != 0);
    if (i > 0) load16(xq, qrow, lo, P.V, P.vec != 0);
  }
  double x[kEPT];
  double own = 0.0;
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {
    x[e] = active ? resid_at(xp[e], i > 0 ? xq[e] : 0.0f, i, S.m) : 0.0;
    own += x[e];
  }
  double ctot;
  double run = base + block_excl_scan_d(own, S, &ctot);
  int cpos = INT_MAX, lastpos = -1;
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {
    const int v = lo + e;
    if (active && v < P.V) {
      if (x[e] > 0.0) lastpos = v;
      run += x[e];
      if (cpos == INT_MAX && run > T) cpos = v;
    }
  }
  const int wcp = wave_min(cpos), wlp = wave_max_i(lastpos);
  if (lane == 0) {
    S.iscan[w] = wcp;
    S.ilast[w] = wlp;
  }
  __syncthreads();
  if (t == 0) {
    int best = INT_MAX, lp = -1;
    for (int k = 0; k < kWaves; ++k) {
      best = min(best, S.iscan[k]);
      lp = max(lp, S.ilast[k]);
    }
    S.tok = best != INT_MAX ? best : lp;
  }
  __syncthreads();
  return S.tok;
}

enum : int { kTry = 0, kAccepted = 1, kRejected = 2, kNoChild = 3 };

__global__ __launch_bounds__(kThreads) void tree_sample_kernel(TreeSampleParams P) {
  __shared__ Shared S;
  const int b = blockIdx.x / P.W, w = blockIdx.x % P.W, t = threadIdx.x;
  const int N = P.N, V = P.V;
  const size_t rowb = static_cast<size_t>(b) * N;
  const float *pb = P.p + rowb * V;
  const float *qb = P.q + rowb * V;
  // the tree, its drafts and uniforms; every lane checks its own node's links
  bool ok = true;
  if (t < N) {
    const int fc = P.first_child[rowb + t], ns = P.next_sibling[rowb + t];
    S.fc[t] = fc;
    S.ns[t] = ns;
    S.d[t] = P.draft[rowb + t];
    S.u[t] = P.u[rowb + t];
    ok = (fc == -1 || (fc > t && fc < N)) && (ns == -1 || (ns > t && ns < N));
  }
  const bool valid = __syncthreads_and(ok);
  const int rem = P.remaining ? P.remaining[b] : -1;   // negative: no budget
  int st = valid ? 0 : SPEC_ST_BAD_STATE;
  int e = 0, acc = 0;
  double fmass = 0.0;
  int ps = 0;                                 // passes so far (each has its own slots)
  bool timed_out = false;
  auto slots_of = [&](int pass) { return P.slots + (static_cast<size_t>(b) * N + pass) * P.chunks; };
  if (valid && rem != 0) {
    int cur = 0;
    int buf = 0;                              // part[buf] holds the current residual's chunk masses
    if (t == 0) S.nodes[0] = 0;
    int nnodes = 1;
    bool done = false;
    while (!done) {
      const float *prow = pb + static_cast<size_t>(cur) * V;
      const float *qrow = qb + static_cast<size_t>(cur) * V;
      int i = 0;                              // rejections at this node (the current residual R_i)
      int child = S.fc[cur];
      int accepted = -1;
      while (child != -1) {
        // lane 0 decides the try of `child` (uniform result through LDS)
        if (t == 0) {
          const int x = S.d[child];
          int s = 0;
          bool yes = false;
          if (x < 0 || x >= V) {
            s |= SPEC_ST_DRAFT_OOR;
          } else {
            const float px = prow[x], qx = qrow[x];
            if (i == 0) {
              if (!isfinite(px) || !isfinite(qx)) s |= SPEC_ST_NONFINITE;
              float a;
              if (qx == 0.0f) {
                a = px > 0.0f ? 1.0f : 0.0f;
                s |= SPEC_ST_Q_ZERO;
              } else {
                const float ratio = __fdiv_rn(px, qx);
                a = ratio < 1.0f ? ratio : 1.0f;
              }
              yes = S.u[child] < a;
            } else {
              yes = accept_resid(resid_at(px, qx, i, S.m), S.m[i], qx, S.u[child], &s);
            }
          }
          S.flag = (yes ? 1 : 0) | (s << 1);
        }
        __syncthreads();
        const int f = S.flag;
        __syncthreads();
        st |= f >> 1;
        if (f & 1) {
          accepted = child;
          break;
        }
        // rejected: the chunk masses and mass of R_{i+1} into the other buffer
        const double mn = residual_pass(P, prow, qrow, i + 1, S, S.part[buf ^ 1], w, slots_of(ps), &timed_out);
        ++ps;
        if (timed_out) {                      // outputs unspecified; every wait still ends
          st |= SPEC_ST_INCOMPLETE;
          done = true;
          break;
        }
        if (!isfinite(mn)) {                  // the round emits token 0 and stops
          st |= SPEC_ST_NONFINITE;
          if (t == 0) S.out[e] = 0;
          ++e;
          fmass = mn;
          done = true;
          break;
        }
        if (mn > 0.0) {
          ++i;
          if (t == 0) S.m[i] = mn;
          buf ^= 1;
          __syncthreads();
        } else {
          st |= SPEC_ST_RESID_ZERO;           // the residual stays R_i
        }
        child = S.ns[child];
      }
      if (done) break;
      if (accepted != -1) {
        const int x = S.d[accepted];
        if (t == 0) S.out[e] = x;
        ++e;
        ++acc;
        if ((P.eos >= 0 && x == P.eos) || e == rem) break;
        if (t == 0) S.nodes[nnodes] = accepted;
        ++nnodes;
        cur = accepted;
        continue;
      }
      // no child accepted, or a leaf: one draw from the current residual
      double Stot;
      if (i == 0) {
        Stot = residual_pass(P, prow, qrow, 0, S, S.part[buf], w, slots_of(ps), &timed_out);
        ++ps;
        if (timed_out) {
          st |= SPEC_ST_INCOMPLETE;
          break;
        }
      } else {
        Stot = S.m[i];
      }
      int tok;
      if (!isfinite(Stot)) {
        st |= SPEC_ST_NONFINITE;
        tok = 0;
      } else if (!(Stot > 0.0)) {
        st |= SPEC_ST_RESID_ZERO;
        tok = 0;
      } else {
        tok = draw_token(P, prow, qrow, i, S, S.part[buf], Stot, S.u[0]);
      }
      if (t == 0) S.out[e] = tok;
      ++e;
      fmass = Stot;
      done = true;
    }
  }
  __syncthreads();
  if (w > 0) {                                // every read of this sequence's slots is done
    if (t == 0) __hip_atomic_store(P.done + static_cast<size_t>(b) * P.W + w, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // member 0: outputs (tokens and kept nodes -1 padded, counts, mass, status)
  if (t < N) {
    P.out_tokens[rowb + t] = t < e ? S.out[t] : -1;
    P.path[rowb + t] = t < e ? S.nodes[t] : -1;
  }
  if (t == 0) {
    P.accept_len[b] = acc;
    P.emit_count[b] = e;
    if (P.final_mass) P.final_mass[b] = fmass;
    if (P.status) P.status[b] = st;
  }
  if (P.W > 1) {
    // once every other member is done with the slots, they and the flags
    // return to zero for the next call (bounded wait)
    int32_t *dn = P.done + static_cast<size_t>(b) * P.W;
    int polls = 0;
    while (true) {
      const bool present = t == 0 || t >= P.W || load_agent(dn + t) != 0;
      if (__syncthreads_and(present)) break;
      if (++polls >= kMaxPolls) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (t > 0 && t < P.W) dn[t] = 0;
    unsigned long long *sl = slots_of(0);
    for (size_t f = t; f < static_cast<size_t>(ps) * P.chunks; f += kThreads) sl[f] = 0ull;
  }
}

// Emit offsets of the batch: one workgroup, after the verification launch.
__global__ __launch_bounds__(kThreads) void tree_sample_offsets_kernel(const int32_t *emit_count,
                                                                       int32_t *emit_offsets, int B) {
  __shared__ int sh[kWaves + 1];
  block_offsets(emit_count, emit_offsets, B, sh);
}

inline int tree_sample_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// Workgroups per sequence: up to 16 while the whole grid fits one workgroup per
// CU on half of the chip (so every member of a sequence is resident at once)
// and the slots stay within 64 MB; else 1 (no workspace).
inline int tree_sample_members(int B, int N, int chunks) {
  if (B > kMaxCoopGroups / 2) return 1;
  if (static_cast<long long>(B) * N * chunks > kMaxCoopSlots) return 1;
  return max(1, min(min(kMaxMembers, kMaxCoopGroups / B), chunks));
}

struct TreeSampleWs {
  size_t slots, done, total;
};
inline TreeSampleWs tree_sample_ws(int B, int N, int chunks, int W) {
  TreeSampleWs l;
  l.slots = 0;
  l.done = round_up(static_cast<size_t>(B) * N * chunks * 8, 256);
  l.total = l.done + round_up(static_cast<size_t>(B) * W * 4, 256);
  return l;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_tree_sample_workspace_bytes(int B, int N, int V) {
  if (B < 1 || N < 1 || V < 1 || N > SPEC_TREE_MAX_N || V >= INT32_MAX - kChunk) return 0;
  const int chunks = tree_sample_chunks(V);
  if (chunks > kMaxChunks) return 0;
  const int W = tree_sample_members(B, N, chunks);
  return W > 1 ? tree_sample_ws(B, N, chunks, W).total : 0;
}

extern "C" int spec_verify_tree_sample(const float *p, const float *q, const int32_t *draft,
                                       const int32_t *first_child, const int32_t *next_sibling,
                                       const float *uniforms, int B, int N, int V, int32_t eos_id,
                                       const int32_t *remaining, int32_t *accept_len, int32_t *emit_count,
                                       int32_t *out_tokens, int32_t *path, int32_t *emit_offsets,
                                       double *final_mass, int32_t *status, void *ws, size_t ws_bytes,
                                       spec_stream_t stream) {
  if (!p || !q || !draft || !first_child || !next_sibling || !uniforms || !accept_len || !emit_count ||
      !out_tokens || !path)
    return SPEC_EINVAL;
  if (B < 1 || N < 1 || V < 1 || V >= INT32_MAX - kChunk) return SPEC_EINVAL;
  if (N > SPEC_TREE_MAX_N) return SPEC_ECAPACITY;
  const int chunks = tree_sample_chunks(V);
  if (chunks > kMaxChunks) return SPEC_ECAPACITY;
  if (!aligned(p, 4) || !aligned(q, 4) || !aligned(uniforms, 4)) return SPEC_EINVAL;
  const size_t rows = static_cast<size_t>(B) * N;
  const size_t nrow = rows * V * 4, nb = static_cast<size_t>(B) * 4, nbn = rows * 4;
  // with a workspace, up to 16 workgroups share each sequence's passes
  const int W = ws ? tree_sample_members(B, N, chunks) : 1;
  const TreeSampleWs lay = tree_sample_ws(B, N, chunks, W);
  if (W > 1 && (ws_bytes < lay.total || !aligned(ws, 256))) return SPEC_EWORKSPACE;
  const size_t wsn = W > 1 ? lay.total : 0;
  const void *ins[] = {p, q, draft, first_child, next_sibling, uniforms, remaining, W > 1 ? ws : nullptr};
  const size_t in_n[] = {nrow, nrow, nbn, nbn, nbn, nbn, nb, wsn};
  const void *outs[] = {accept_len, emit_count, out_tokens, path, emit_offsets, final_mass, status};
  const size_t out_n[] = {nb, nb, nbn, nbn, nb + 4, static_cast<size_t>(B) * 8, nb};
  for (int i = 0; i < 7; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 7; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }
  TreeSampleParams P;
  P.p = p;
  P.q = q;
  P.draft = draft;
  P.first_child = first_child;
  P.next_sibling = next_sibling;
  P.u = uniforms;
  P.B = B;
  P.N = N;
  P.V = V;
  P.chunks = chunks;
  P.vec = (V % 4 == 0) && aligned(p, 16) && aligned(q, 16);
  P.eos = eos_id;
  P.remaining = remaining;
  P.accept_len = accept_len;
  P.emit_count = emit_count;
  P.out_tokens = out_tokens;
  P.path = path;
  P.emit_offsets = emit_offsets;
  P.final_mass = final_mass;
  P.status = status;
  P.W = W;
  unsigned char *wb = static_cast<unsigned char *>(ws);
  P.slots = W > 1 ? reinterpret_cast<unsigned long long *>(wb + lay.slots) : nullptr;
  P.done = W > 1 ? reinterpret_cast<int32_t *>(wb + lay.done) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(tree_sample_kernel, dim3(static_cast<unsigned>(B * W)), dim3(kThreads), 0, s, P);
  if (emit_offsets)
    hipLaunchKernelGGL(tree_sample_offsets_kernel, dim3(1), dim3(kThreads), 0, s, emit_count, emit_offsets, B);
  return launch_status();
}
