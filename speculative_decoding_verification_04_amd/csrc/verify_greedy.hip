// Greedy verification of a batch of speculative rounds (gfx950).
//
// What it computes follows the greedy commitment of the zero-to-sglang
// "Chapter 10 Speculative Decoding (Code Walkthrough)" 4.1 and the BatchVerify
// description in the "Correctness Forensics for Batch Speculative Decoding"
// summary, App. D; the row alignment (row j verifies draft j, row k is the
// bonus row) is the walkthrough's 3.3 table.
//
// Design.  The logits are the only large input (B*(k+1)*V elements), so the
// step is one streaming pass over them, bound by HBM bandwidth, followed by a
// tiny commit pass.
//   * greedy_chunk_kernel: each row is cut into chunks of kThreads*VEC*U
//     elements; one workgroup per (row, chunk) loads its chunk with 16-byte
//     non-temporal loads (U in flight per lane).  The chunk maximum comes from
//     plain max instructions, DPP lane moves inside each wave and LDS across
//     waves; then only the lanes holding it search their own elements for its
//     first index (an LDS minimum picks the lowest), and one 64-bit key is
//     stored (value order high, UINT32_MAX - index low; the largest key is
//     the argmax at the lowest index).  Searching in every lane, or reducing
//     64-bit keys through LDS permutes, measured about 0.5 us slower.  No workgroup waits for another: cross-workgroup completion
//     tickets cost far more than this whole pass on a multi-XCD part (device-
//     scope atomics on one address serialise, and waiting on them holds the
//     CU's wave slots), so the kernel boundary is the synchronisation.
//   * greedy_commit_kernel: one workgroup; one lane per row folds that row's
//     chunk keys in registers, then one lane per sequence walks its drafts and
//     writes its outputs, and the emit counts are scanned into offsets, a tile
//     of sequences at a time.
#include "common.h"

namespace specv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <bool BF16>
struct GreedyTraits;
template <>
struct GreedyTraits<true> {
  static constexpr int ELT = 2, VEC = 8, U = 4;
};
template <>
struct GreedyTraits<false> {
  static constexpr int ELT = 4, VEC = 4, U = 4;
};

struct GreedyParams {
  const unsigned char *logits;
  int B, k, V, chunks, chunk_elems;
  const int32_t *draft;
  int32_t eos;
  const int32_t *remaining;
  int32_t *accept_len, *emit_count, *out_tokens, *emit_offsets, *status;
  uint64_t *keys;     // [B*(k+1)*chunks]
  // tree verification only (k + 1 = N nodes per sequence)
  const int32_t *first_child, *next_sibling;
  int32_t *path;
};

inline size_t greedy_ws_bytes(int B, int k, int chunks) {
  return round_up(static_cast<size_t>(B) * (k + 1) * chunks * sizeof(uint64_t), 256);
}

template <bool BF16>
inline int greedy_chunk_elems() {
  using Tr = GreedyTraits<BF16>;
  return kThreads * Tr::VEC * Tr::U;
}

inline int greedy_chunks(int V, spec_dtype dt) {
  const int ce = dt == SPEC_BF16 ? greedy_chunk_elems<true>() : greedy_chunk_elems<false>();
  return (V + ce - 1) / ce;
}

template <bool BF16>
__device__ inline float load_elem(const unsigned char *p, int i) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(p)[i]) << 16);
  } else {
    return reinterpret_cast<const float *>(p)[i];
  }
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte streaming load: the logits are read exactly once.
__device__ inline uint4 stream_load(const unsigned char *p) {
  const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

template <bool BF16>
__device__ inline uint4 neg_inf_vec() {
  const uint32_t w = BF16 ? 0xFF80FF80u : 0xFF800000u;
  return make_uint4(w, w, w, w);
}

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool BF16>
__device__ inline float vec_max(uint4 x) {
  if constexpr (BF16) {
    float a = fmaxf(fmaxf(lo_bf16(x.x), hi_bf16(x.x)), lo_bf16(x.y));
    float b = fmaxf(fmaxf(hi_bf16(x.y), lo_bf16(x.z)), hi_bf16(x.z));
    float c = fmaxf(lo_bf16(x.w), hi_bf16(x.w));
    return fmaxf(fmaxf(a, b), c);
  } else {
    return fmaxf(fmaxf(__uint_as_float(x.x), __uint_as_float(x.y)),
                 fmaxf(__uint_as_float(x.z), __uint_as_float(x.w)));
  }
}

// Position (0..VEC-1) of the first element equal to m, or VEC.
template <bool BF16>
__device__ inline int vec_find(uint4 x, float m) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  int q = BF16 ? 8 : 4;
  // scanned from the back so the first match wins; no early exit (no branches)
  if constexpr (BF16) {
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      q = hi_bf16(w[i]) == m ? 2 * i + 1 : q;
      q = lo_bf16(w[i]) == m ? 2 * i : q;
    }
  } else {
#pragma unroll
    for (int i = 3; i >= 0; --i) q = __uint_as_float(w[i]) == m ? i : q;
  }
  return q;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void greedy_chunk_kernel(GreedyParams P) {
  using Tr = GreedyTraits<BF16>;
  constexpr int ELT = Tr::ELT, VEC = Tr::VEC, U = Tr::U;
  __shared__ float sh_max[kWaves];
  __shared__ int sh_first;

  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int row = blockIdx.x / P.chunks;
  const int c = blockIdx.x - row * P.chunks;
  const unsigned char *rowp = P.logits + static_cast<size_t>(row) * P.V * ELT;
  // Elements before the row's first 16-byte boundary are handled one per lane
  // by chunk 0; the body starts aligned.
  const int head = min(P.V, static_cast<int>(((16u - (reinterpret_cast<uintptr_t>(rowp) & 15u)) & 15u) / ELT));
  const int s = head + c * P.chunk_elems;
  const int e = min(P.V, s + P.chunk_elems);
  const int nv = e > s ? (e - s) / VEC : 0;
  const int ntail = e > s ? (e - s) - nv * VEC : 0;

  const bool has_head = (c == 0) && (t < head);
  const bool has_tail = t < ntail;
  float hv = -INFINITY, tv = -INFINITY;
  if (has_head) hv = load_elem<BF16>(rowp, t);
  uint4 buf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = t + u * kThreads;
    buf[u] = vi < nv ? stream_load(rowp + static_cast<size_t>(s + vi * VEC) * ELT) : neg_inf_vec<BF16>();
  }
  if (has_tail) tv = load_elem<BF16>(rowp, s + nv * VEC + t);

  // Lane maximum (the -inf filler of missing vectors cannot exceed it unless
  // the lane holds no element at all), then the chunk maximum: DPP inside each
  // wave, LDS across the waves.
  float lmax = fmaxf(hv, tv);
#pragma unroll
  for (int u = 0; u < U; ++u) lmax = fmaxf(lmax, vec_max<BF16>(buf[u]));
  const float wm = wave_max_dpp(lmax);
  if (t == 0) sh_first = INT_MAX;
  if (lane == 0) sh_max[w] = wm;
  __syncthreads();
  float bmax = sh_max[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) bmax = fmaxf(bmax, sh_max[i]);

  // Only lanes holding the chunk maximum look for its first index among their
  // own elements, visited in increasing index order (head, vectors u = 0..U-1,
  // tail); an LDS minimum across those lanes gives the chunk's first index.
  if (lmax == bmax) {
    int cand = INT_MAX;
    if (has_tail && tv == bmax) cand = s + nv * VEC + t;
#pragma unroll
    for (int u = U - 1; u >= 0; --u) {
      const int vi = t + u * kThreads;
      const int q = vec_find<BF16>(buf[u], bmax);
      if (vi < nv && q < VEC) cand = s + vi * VEC + q;
    }
    if (has_head && hv == bmax) cand = t;
    if (cand != INT_MAX) atomicMin(&sh_first, cand);
  }
  __syncthreads();
  if (t == 0)
    P.keys[static_cast<size_t>(row) * P.chunks + c] = sh_first == INT_MAX ? 0ull : argmax_key(bmax, sh_first);
}

constexpr int kCommitThreads = 1024;
constexpr int kCommitRows = 1024;   // row keys folded per tile (LDS)
constexpr int kKeysPerThread = 16;  // chunk keys in flight per lane
static_assert(kCommitRows == kCommitThreads, "one row (and at most one draft) per lane of a tile");

// One workgroup.  Per tile of sequences, every global read (chunk keys, drafts,
// budgets) is issued at once into LDS; the walk then runs from LDS only.
__global__ __launch_bounds__(kCommitThreads) void greedy_commit_kernel(GreedyParams P) {
  __shared__ unsigned long long sh_row[kCommitRows];
  __shared__ int sh_d[kCommitRows];
  __shared__ int sh_rem[kCommitRows];
  __shared__ int sh_scan[kCommitThreads / kWave + 1];
  const int t = threadIdx.x;
  const int kp1 = P.k + 1;
  const int per_tile = kCommitRows / kp1;          // sequences per tile (k <= SPEC_MAX_K keeps this >= 8)
  int carry = 0;
  for (int s0 = 0; s0 < P.B; s0 += per_tile) {
    const int ns = min(per_tile, P.B - s0);
    const int nrows = ns * kp1;
    // one round trip: drafts, budgets and every chunk key are requested before
    // any is used (into registers; LDS is written once all have landed); lane
    // r folds row r's keys (no LDS atomics).  A tile holds at most one draft
    // and one row per lane: ns * k < ns * (k + 1) <= kCommitRows.
    const uint64_t *kb = P.keys + static_cast<size_t>(s0) * kp1 * P.chunks;
    const bool has_d = t < ns * P.k, has_r = t < nrows;
    const int dv = has_d ? P.draft[static_cast<size_t>(s0) * P.k + t] : 0;
    const int rv = t < ns && P.remaining ? P.remaining[s0 + t] : -1;   // negative: no budget
    uint64_t best = 0ull;
    if (has_r) {
      const uint64_t *rk = kb + static_cast<size_t>(t) * P.chunks;
      for (int c0 = 0; c0 < P.chunks; c0 += kKeysPerThread) {
        uint64_t kr[kKeysPerThread];
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) kr[q] = c0 + q < P.chunks ? rk[c0 + q] : 0ull;
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) best = kr[q] > best ? kr[q] : best;
      }
    }
    if (has_d) sh_d[t] = dv;
    if (t < ns) sh_rem[t] = rv;
    if (has_r) sh_row[t] = best;
    __syncthreads();
    int cnt = 0;
    if (t < ns) {
      const int b = s0 + t;
      const int *d = sh_d + t * P.k;
      int32_t *out = P.out_tokens + static_cast<size_t>(b) * kp1;
      const unsigned long long *rk = sh_row + t * kp1;
      const int rem = sh_rem[t];
      int st = 0;
      for (int j = 0; j < P.k; ++j)
        if (d[j] < 0 || d[j] >= P.V) st |= SPEC_ST_DRAFT_OOR;
      int acc = 0;
      if (rem != 0) {
        bool stop = false;
        for (int j = 0; j < P.k && !stop; ++j) {
          const int tj = argmax_key_index(rk[j]);
          out[cnt++] = tj;
          const bool match = tj == d[j];
          acc += match;
          if ((P.eos >= 0 && tj == P.eos) || cnt == rem || !match) stop = true;
        }
        if (!stop) out[cnt++] = argmax_key_index(rk[P.k]);
      }
      for (int i = cnt; i < kp1; ++i) out[i] = -1;
      P.accept_len[b] = acc;
      P.emit_count[b] = cnt;
      if (P.status) P.status[b] = st;
    }
    if (P.emit_offsets) {
      int total;
      const int ex = block_excl_scan(t < ns ? cnt : 0, sh_scan, &total);
      if (t < ns) P.emit_offsets[s0 + t] = carry + ex;
      carry += total;
    }
    __syncthreads();
  }
  if (P.emit_offsets && t == 0) P.emit_offsets[P.B] = carry;
}

// Greedy verification of a candidate tree (one logit row per node, rows from
// greedy_chunk_kernel's keys).  One workgroup; per tile of sequences every
// global read (keys, drafts, links, budgets) is issued first, then one lane
// per sequence walks its tree from LDS: take the argmax of the current node's
// row, accept the first child (in sibling order) proposing it, else emit it
// and stop.  Links must point forward inside the tree, so a walk visits at
// most N nodes and every sibling scan ends.
constexpr int kTreeRows = 1024;
static_assert(kTreeRows == kCommitThreads, "one lane per tree node of a tile");

// One workgroup; tiles of whole sequences, one lane per node (row).  Each lane
// folds its row's chunk keys into the row's argmax, checks its own links and
// draft id, and finds which of its children (if any) proposes that argmax;
// one lane per sequence then only follows those precomputed edges from the
// root, and the emitted tokens and path are written back by all lanes.
__global__ __launch_bounds__(kCommitThreads) void tree_commit_kernel(GreedyParams P) {
  __shared__ int sh_d[kTreeRows];     // draft ids; after the walk: emitted tokens
  __shared__ int sh_fc[kTreeRows];    // first child; after the walk: path nodes
  __shared__ int sh_ns[kTreeRows];
  __shared__ int sh_tok[kTreeRows];   // argmax of each node's row
  __shared__ int sh_nxt[kTreeRows];   // child proposing that argmax, or -1
  __shared__ int sh_st[kTreeRows];    // per-sequence status bits
  __shared__ int sh_cnt[kTreeRows];   // per-sequence budget, then emitted count
  __shared__ int sh_scan[kCommitThreads / kWave + 1];
  const int t = threadIdx.x;
  const int N = P.k + 1;
  const int per_tile = kTreeRows / N;                // N <= SPEC_TREE_MAX_N keeps this >= 4
  int carry = 0;
  for (int s0 = 0; s0 < P.B; s0 += per_tile) {
    const int nseq = min(per_tile, P.B - s0);
    const int nrows = nseq * N;
    const size_t r0 = static_cast<size_t>(s0) * N;
    const bool row = t < nrows;
    const int seq = t / N, node = t - seq * N, base = seq * N;
    int d = 0, fc = -1, ns = -1;
    uint64_t best = 0ull;
    if (row) {
      d = P.draft[r0 + t];
      fc = P.first_child[r0 + t];
      ns = P.next_sibling[r0 + t];
      const uint64_t *rk = P.keys + (r0 + t) * P.chunks;
      for (int c0 = 0; c0 < P.chunks; c0 += kKeysPerThread) {
        uint64_t kr[kKeysPerThread];
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) kr[q] = c0 + q < P.chunks ? rk[c0 + q] : 0ull;
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) best = kr[q] > best ? kr[q] : best;
      }
    }
    if (t < nseq) {
      sh_st[t] = 0;
      sh_cnt[t] = P.remaining ? P.remaining[s0 + t] : -1;
    }
    const int tok = argmax_key_index(best);
    if (row) {
      sh_d[t] = d;
      sh_fc[t] = fc;
      sh_ns[t] = ns;
      sh_tok[t] = tok;
    }
    __syncthreads();
    if (row) {
      int bits = 0;
      if (node > 0 && (d < 0 || d >= P.V)) bits |= SPEC_ST_DRAFT_OOR;
      if ((fc != -1 && (fc <= node || fc >= N)) || (ns != -1 && (ns <= node || ns >= N)))
        bits |= SPEC_ST_BAD_STATE;
      if (bits) atomicOr(&sh_st[seq], bits);
    }
    __syncthreads();
    if (row) {
      int c = -1;
      if (!(sh_st[seq] & SPEC_ST_BAD_STATE)) {        // every link of this tree points forward
        c = fc;
        while (c != -1 && sh_d[base + c] != tok) c = sh_ns[base + c];
      }
      sh_nxt[t] = c;
    }
    __syncthreads();
    int cnt = 0;
    if (t < nseq) {
      const int b = s0 + t;
      const int sb = t * N;
      const int st = sh_st[t];
      const int rem = sh_cnt[t];
      int acc = 0;
      if (!(st & SPEC_ST_BAD_STATE) && rem != 0) {
        int cur = 0;
        while (true) {
          const int tk = sh_tok[sb + cur];
          const int c = sh_nxt[sb + cur];
          sh_d[sb + cnt] = tk;                          // drafts and links are no longer read:
          sh_fc[sb + cnt] = cur;                        // their rows now hold tokens and path
          ++cnt;
          if (c != -1) ++acc;
          if ((P.eos >= 0 && tk == P.eos) || cnt == rem || c == -1) break;
          cur = c;
        }
      }
      sh_cnt[t] = cnt;
      P.accept_len[b] = acc;
      P.emit_count[b] = cnt;
      if (P.status) P.status[b] = st;
    }
    __syncthreads();
    if (row) {
      const bool kept = node < sh_cnt[seq];
      P.out_tokens[r0 + t] = kept ? sh_d[t] : -1;
      P.path[r0 + t] = kept ? sh_fc[t] : -1;
    }
    if (P.emit_offsets) {
      int total;
      const int ex = block_excl_scan(t < nseq ? cnt : 0, sh_scan, &total);
      if (t < nseq) P.emit_offsets[s0 + t] = carry + ex;
      carry += total;
    }
    __syncthreads();
  }
  if (P.emit_offsets && t == 0) P.emit_offsets[P.B] = carry;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_greedy_workspace_bytes(int B, int k, int V, spec_dtype dt) {
  if (B < 1 || k < 1 || V < 1 || k > SPEC_MAX_K) return 0;
  return greedy_ws_bytes(B, k, greedy_chunks(V, dt));
}

extern "C" int spec_verify_greedy(const void *logits, spec_dtype dt, int B, int k, int V,
                                  const int32_t *draft, int32_t eos_id, const int32_t *remaining,
                                  int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                                  int32_t *emit_offsets, int32_t *status, void *ws,
                                  size_t ws_bytes, spec_stream_t stream) {
  if (!logits || !draft || !accept_len || !emit_count || !out_tokens || !ws) return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (B < 1 || k < 1 || V < 1 || V >= INT32_MAX - 1) return SPEC_EINVAL;
  if (k > SPEC_MAX_K) return SPEC_ECAPACITY;
  const size_t elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(logits, elt)) return SPEC_EINVAL;
  const int chunks = greedy_chunks(V, dt);
  const long long nblocks = static_cast<long long>(B) * (k + 1) * chunks;
  if (nblocks >= INT32_MAX) return SPEC_EINVAL;
  const size_t wsb = greedy_ws_bytes(B, k, chunks);
  if (ws_bytes < wsb || !aligned(ws, 256)) return SPEC_EWORKSPACE;

  const size_t nl = static_cast<size_t>(B) * (k + 1) * V * elt;
  const void *ins[] = {logits, draft, remaining, ws};
  const size_t in_n[] = {nl, static_cast<size_t>(B) * k * 4, static_cast<size_t>(B) * 4, wsb};
  const void *outs[] = {accept_len, emit_count, out_tokens, emit_offsets, status};
  const size_t out_n[] = {static_cast<size_t>(B) * 4, static_cast<size_t>(B) * 4,
                          static_cast<size_t>(B) * (k + 1) * 4, static_cast<size_t>(B + 1) * 4,
                          static_cast<size_t>(B) * 4};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }

  GreedyParams P;
  P.logits = static_cast<const unsigned char *>(logits);
  P.B = B;
  P.k = k;
  P.V = V;
  P.chunks = chunks;
  P.chunk_elems = dt == SPEC_BF16 ? greedy_chunk_elems<true>() : greedy_chunk_elems<false>();
  P.draft = draft;
  P.eos = eos_id;
  P.remaining = remaining;
  P.accept_len = accept_len;
  P.emit_count = emit_count;
  P.out_tokens = out_tokens;
  P.emit_offsets = emit_offsets;
  P.status = status;
  P.keys = static_cast<uint64_t *>(ws);
  P.first_child = P.next_sibling = nullptr;
  P.path = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dt == SPEC_BF16)
    hipLaunchKernelGGL(greedy_chunk_kernel<true>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL(greedy_chunk_kernel<false>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  hipLaunchKernelGGL(greedy_commit_kernel, dim3(1), dim3(kCommitThreads), 0, s, P);
  return launch_status();
}

extern "C" size_t spec_verify_tree_workspace_bytes(int B, int N, int V, spec_dtype dt) {
  if (B < 1 || N < 1 || V < 1 || N > SPEC_TREE_MAX_N) return 0;
  return greedy_ws_bytes(B, N - 1, greedy_chunks(V, dt));
}

extern "C" int spec_verify_tree(const void *logits, spec_dtype dt, int B, int N, int V,
                                const int32_t *draft, const int32_t *first_child,
                                const int32_t *next_sibling, int32_t eos_id, const int32_t *remaining,
                                int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                                int32_t *path, int32_t *emit_offsets, int32_t *status, void *ws,
                                size_t ws_bytes, spec_stream_t stream) {
  if (!logits || !draft || !first_child || !next_sibling || !accept_len || !emit_count || !out_tokens ||
      !path || !ws)
    return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (B < 1 || N < 1 || V < 1 || V >= INT32_MAX - 1) return SPEC_EINVAL;
  if (N > SPEC_TREE_MAX_N) return SPEC_ECAPACITY;
  const size_t elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(logits, elt)) return SPEC_EINVAL;
  const int chunks = greedy_chunks(V, dt);
  const long long nblocks = static_cast<long long>(B) * N * chunks;
  if (nblocks >= INT32_MAX) return SPEC_EINVAL;
  const size_t wsb = greedy_ws_bytes(B, N - 1, chunks);
  if (ws_bytes < wsb || !aligned(ws, 256)) return SPEC_EWORKSPACE;
  const size_t bn4 = static_cast<size_t>(B) * N * 4, b4 = static_cast<size_t>(B) * 4;
  const void *ins[] = {logits, draft, first_child, next_sibling, remaining, ws};
  const size_t in_n[] = {static_cast<size_t>(B) * N * V * elt, bn4, bn4, bn4, b4, wsb};
  const void *outs[] = {accept_len, emit_count, out_tokens, path, emit_offsets, status};
  const size_t out_n[] = {b4, b4, bn4, bn4, b4 + 4, b4};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }
  GreedyParams P;
  P.logits = static_cast<const unsigned char *>(logits);
  P.B = B;
  P.k = N - 1;
  P.V = V;
  P.chunks = chunks;
  P.chunk_elems = dt == SPEC_BF16 ? greedy_chunk_elems<true>() : greedy_chunk_elems<false>();
  P.draft = draft;
  P.eos = eos_id;
  P.remaining = remaining;
  P.accept_len = accept_len;
  P.emit_count = emit_count;
  P.out_tokens = out_tokens;
  P.emit_offsets = emit_offsets;
  P.status = status;
  P.keys = static_cast<uint64_t *>(ws);
  P.first_child = first_child;
  P.next_sibling = next_sibling;
  P.path = path;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dt == SPEC_BF16)
    hipLaunchKernelGGL(greedy_chunk_kernel<true>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL(greedy_chunk_kernel<false>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  hipLaunchKernelGGL(tree_commit_kernel, dim3(1), dim3(kCommitThreads), 0, s, P);
  return launch_status();
}
