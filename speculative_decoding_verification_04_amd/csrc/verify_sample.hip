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
#include "sample_src.h"

namespace specv {
namespace {

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
// order within a wave, then waves); *total receives the block total.  One
// barrier: `sh` (kWaves doubles) must not be written again before a later
// barrier.
__device__ inline double block_excl_scan_d1(double v, double *sh, double *total) {
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


// Chunk masses travel as 64-bit keys: the mass's bits XOR kMassSentinel.
// The sentinel is a NaN whose low 29 bits are not all zero, a pattern no mass
// here can take (a float32 widened to float64, and any arithmetic on such
// values, gives NaNs with those bits zero), so every published key is nonzero
// and a zero slot means "not yet written".
constexpr unsigned long long kMassSentinel = 0x7FF4000000000001ull;

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
  __shared__ double sh_pre[kThreads];
  __shared__ int sh_scan[2][kWaves];
  __shared__ int sh_last[2][kWaves];
  __shared__ double sh_dscan[3][kWaves + 1];

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
    if (timed_out) {
      st |= SPEC_ST_INCOMPLETE;
    } else {
      typename Src::RowT r = Src::row(P, b, jrow, mode == MODE_RESID);
      const bool vec = P.vec != 0;
      const int per = (nc + kThreads - 1) / kThreads;  // chunks per lane, consecutive
      const int c0 = t * per;
      // total mass and each lane's exclusive prefix over the chunk masses
      double pre = 0.0;
      auto scan_parts = [&](double *sh) {
        double mine = 0.0;
        for (int i = 0; i < per; ++i)
          if (c0 + i < nc) mine += sh_part[c0 + i];
        pre = block_excl_scan_d1(mine, sh, &S);
      };
      scan_parts(sh_dscan[0]);
      if (isfinite(S) && !(S > 0.0)) {
        st |= SPEC_ST_RESID_ZERO;
        if (mode == MODE_RESID) {         // fall back to the target row p_j itself
          r.resid = false;
          for (int i = 0; i < nc; ++i) {
            const double part = chunk_mass(r, i, V, vec, sh_red);
            if (t == 0) sh_part[i] = part;
          }
          __syncthreads();
          scan_parts(sh_dscan[1]);
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
        sh_pre[t] = pre;
        const int wc = wave_min(cand), wl = wave_max_i(last);
        if (lane == 0) {
          sh_scan[0][w] = wc;
          sh_last[0][w] = wl;
        }
        __syncthreads();
        int cs = INT_MAX, lp = -1;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
          cs = min(cs, sh_scan[0][i]);
          lp = max(lp, sh_last[0][i]);
        }
        if (cs == INT_MAX) cs = lp;
        // mass before chunk cs, added in its owner lane's order
        const int owner = cs / per;
        double base = sh_pre[owner];
        for (int c = owner * per; c < cs; ++c) base += sh_part[c];
        // in-chunk scan in index order: lane t owns kEPT consecutive entries
        const int lo = cs * kChunk + t * kEPT;
        float x[kEPT];
        r.load16(x, lo, V, vec);
        double mine = 0.0;
#pragma unroll
        for (int i = 0; i < kEPT; ++i) mine += static_cast<double>(x[i]);
        double ctot;
        double run = base + block_excl_scan_d1(mine, sh_dscan[2], &ctot);
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
          sh_scan[1][w] = wcp;
          sh_last[1][w] = wlp;
        }
        __syncthreads();
        int best = INT_MAX, lpos = -1;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
          best = min(best, sh_scan[1][i]);
          lpos = max(lpos, sh_last[1][i]);
        }
        tok = best != INT_MAX ? best : lpos;
      }
    }
    // every slot back to zero (ordered before the next call by the launch);
    // issued after the draw's loads, which would otherwise wait for them
    for (int i = t; i < nc; i += kThreads) keys[i] = 0ull;
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
// B * (k+1) target and B * k draft rows, the slice lists, their entries'
// indices and three published words per row (all rewritten by every call),
// then the layout of spec_verify_sample.
struct LogitsWs {
  size_t lists, idx, flags, total;
};
static LogitsWs sample_logits_layout(int B, int k, int V) {
  const int rows = B * (2 * k + 1);
  LogitsWs w;
  w.lists = round_up(static_cast<size_t>(rows) * sizeof(ProcStats), 256);
  w.idx = w.lists + proc_list_bytes(rows, V);
  w.flags = w.idx + proc_list_idx_bytes(rows);
  w.total = w.flags + round_up(static_cast<size_t>(rows) * 3 * sizeof(unsigned long long), 256);
  return w;
}
static size_t sample_logits_stats_bytes(int B, int k, int V) { return sample_logits_layout(B, k, V).total; }

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
  const LogitsWs lw = sample_logits_layout(B, k, V);
  (void)hipGetLastError();
  // through the slice lists (top-k, or top-p alone): the slice launches,
  // then statistics and verification in one launch
  if (launch_sample_logits_lists(P, bf16, top_k, top_p, stats, wb + lw.lists,
                                reinterpret_cast<int32_t *>(wb + lw.idx),
                                reinterpret_cast<unsigned long long *>(wb + lw.flags), s))
    return launch_status();
  launch_proc_stats(target_logits, draft_logits, B * (k + 1), static_cast<int>(rows), V, bf16, P.invT,
                    top_k, top_p, stats, nullptr, wb + lw.lists, s);
  const dim3 grid = sample_grid(B, chunks, emit_offsets), blk(kThreads);
  if (bf16)
    hipLaunchKernelGGL(sample_verify_kernel<LogitSrc<true>>, grid, blk, 0, s, P);
  else
    hipLaunchKernelGGL(sample_verify_kernel<LogitSrc<false>>, grid, blk, 0, s, P);
  return launch_status();
}
