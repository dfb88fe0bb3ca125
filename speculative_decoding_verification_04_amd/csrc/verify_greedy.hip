// Greedy verification of a batch of speculative rounds (gfx950).
//
// What it computes follows the greedy commitment of the zero-to-sglang
// "Chapter 10 Speculative Decoding (Code Walkthrough)" 4.1 and the BatchVerify
// description in the "Correctness Forensics for Batch Speculative Decoding"
// summary, App. D; the row alignment (row j verifies draft j, row k is the
// bonus row) is the walkthrough's 3.3 table.
//
// Design.  The logits are the only large input (B*(k+1)*V elements), so the
// step is one streaming pass over them, bound by HBM bandwidth, plus a tiny
// commit.  One launch does both:
//   * producer workgroups (one per (row, chunk of kThreads*VEC*U elements))
//     load their chunk with 16-byte non-temporal loads (U in flight per lane).
//     The chunk maximum comes from plain max instructions, DPP lane moves
//     inside each wave and LDS across waves; only the lanes holding it search
//     their own elements for its first index (an LDS minimum picks the
//     lowest).  The chunk's 64-bit key (value order high, UINT32_MAX - index
//     low; the largest key is the argmax at the lowest index) is published
//     with one agent-scope store into its workspace slot.  A published key is
//     never 0 (an empty chunk publishes 1), so a slot is its own flag.
//   * workgroup 0, the finisher, walks the batch in tiles of sequences: it
//     polls a tile's slots with agent-scope loads (one round of loads per
//     poll, only missing slots re-read) and, while the next tile's slots and
//     drafts are already being loaded, commits the tile in LDS with one lane
//     per row: fold the row's chunk keys, test its stop conditions (mismatch,
//     EOS) with an LDS minimum per sequence, then one lane per sequence applies
//     the budget, counts the accepted drafts and scans the emit counts, and
//     the rows write their tokens.  Finally it returns every slot it read to
//     0 (the workspace stays zero-filled between calls).
// Producers never wait: the finisher is one workgroup whose wait ends when
// every producer has published, and producers depend on nothing.  Device-
// scope atomics on shared counters are avoided altogether (on a multi-XCD
// part they serialise per address).  Sequences whose rows need more chunk
// keys than one finisher tile holds fall back to two launches: the streaming
// kernel, then a one-workgroup commit (tree verification uses the same
// streaming kernel with its own commit).
#include "common.h"

#include <mutex>

namespace specv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr uint64_t kEmptyKey = 1ull;   // published by a chunk with no elements (below every real key)

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
  uint64_t *keys;     // [B*(k+1)*chunks]; zero between calls (the slot flags)
  int nprod;          // producer workgroups of the single-launch path
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

// One producer: the key of chunk c of row `row`.  PUBLISH stores it with an
// agent-scope store (visible to the finisher of the same launch); otherwise
// with a plain store (read by a later kernel).
template <bool BF16, bool PUBLISH>
__device__ inline void stream_chunk(const GreedyParams &P, int blk) {
  using Tr = GreedyTraits<BF16>;
  constexpr int ELT = Tr::ELT, VEC = Tr::VEC, U = Tr::U;
  __shared__ float sh_max[kWaves];
  __shared__ int sh_first;

  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int row = blk / P.chunks;
  const int c = blk - row * P.chunks;
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
  if (t == 0) {
    const uint64_t key = sh_first == INT_MAX ? kEmptyKey : argmax_key(bmax, sh_first);
    uint64_t *slot = P.keys + static_cast<size_t>(row) * P.chunks + c;
    if constexpr (PUBLISH) __hip_atomic_store(slot, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *slot = key;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void greedy_chunk_kernel(GreedyParams P) {
  stream_chunk<BF16, false>(P, blockIdx.x);
}

// ---------------------------------------------------------------- commit ----
// The finisher commits a tile of sequences in LDS: kTileKeys chunk keys per
// tile (at most kTileSeq sequences), rows = ns * (k + 1) <= kTileKeys / chunks.
// Its last wave only stores results; the other waves only load.  A wave's
// memory counter covers its loads and its stores alike, so a wave that waits
// for its loads never waits for stores as well.
constexpr int kTileKeys = 1024;
constexpr int kTileSeq = 256;
constexpr int kLoadLanes = kThreads - kWave;                              // waves 0 .. kWaves-2
constexpr int kKPL = (kTileKeys + kLoadLanes - 1) / kLoadLanes;           // slots per loading lane
static_assert(kTileSeq <= kLoadLanes, "one loading lane per sequence of a tile");

struct TileShared {
  uint64_t key[kTileKeys];   // the tile's chunk keys, row-major
  int tok[kTileKeys];        // argmax of each row
  int d[kTileKeys];          // the tile's drafts (ns * k <= kTileKeys)
  int stop[kTileSeq];        // first row that stops the sequence (LDS minimum)
  int rem[kTileSeq];         // budgets
  int st[kTileSeq];          // status bits
  int e[kTileSeq];           // emit counts
  int acc[kTileSeq];         // accepted drafts
  int off[kTileSeq];         // emit offsets
  int scan[kThreads / kWave + 1];
};

__host__ __device__ inline int tile_sequences(int k, int chunks) {
  const int rows = kTileKeys / chunks;
  return min(kTileSeq, rows / (k + 1));
}

// Commits the ns sequences starting at s0 whose chunk keys, drafts and budgets
// are in LDS (stop[] holds k and st[] the status on entry).  Every lane of the
// workgroup calls it; only the last wave writes global memory.  Returns the
// carry of the emit offsets.
__device__ inline int commit_tile(const GreedyParams &P, TileShared &S, int s0, int ns, int carry) {
  const int t = threadIdx.x, kp1 = P.k + 1, nrows = ns * kp1;
  // one lane per row: fold its chunk keys, then test the row's stop
  // conditions (draft j < k: a mismatch or EOS stops after emitting row j)
  for (int r = t; r < nrows; r += kThreads) {
    const uint64_t *kr = S.key + r * P.chunks;
    uint64_t best = 0ull;
    int c = 0;
    for (; c + 8 <= P.chunks; c += 8) {
      uint64_t x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = kr[c + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) best = x[q] > best ? x[q] : best;
    }
    for (; c < P.chunks; ++c) best = kr[c] > best ? kr[c] : best;
    const int tok = argmax_key_index(best);
    S.tok[r] = tok;
    const int b = r / kp1, j = r - b * kp1;
    if (j < P.k) {
      const int d = S.d[b * P.k + j];
      if (d < 0 || d >= P.V) atomicOr(&S.st[b], SPEC_ST_DRAFT_OOR);
      if (tok != d || (P.eos >= 0 && tok == P.eos)) atomicMin(&S.stop[b], j);
    }
  }
  __syncthreads();
  // one lane per sequence: emitted count (first stop row + 1, capped by the
  // budget) and accepted drafts (every emitted row before the last matched;
  // the last emitted row counts if it matched its draft)
  int cnt = 0;
  if (t < ns) {
    const int rem = S.rem[t];
    cnt = S.stop[t] + 1;
    if (rem >= 0) cnt = min(cnt, rem);
    int acc = 0;
    if (cnt > 0) {
      const int last = cnt - 1;
      acc = last + ((last < P.k && S.tok[t * kp1 + last] == S.d[t * P.k + last]) ? 1 : 0);
    }
    S.e[t] = cnt;
    S.acc[t] = acc;
  }
  int total;
  const int ex = block_excl_scan(t < ns ? cnt : 0, S.scan, &total);   // ends with a barrier
  if (t < ns) S.off[t] = carry + ex;
  __syncthreads();
  // the store wave writes the tile's results
  if (t >= kLoadLanes) {
    const int l = t - kLoadLanes;
    int32_t *out = P.out_tokens + static_cast<size_t>(s0) * kp1;
    for (int r = l; r < nrows; r += kWave) {
      const int b = r / kp1, j = r - b * kp1;
      out[r] = j < S.e[b] ? S.tok[r] : -1;
    }
    for (int i = l; i < ns; i += kWave) {
      P.accept_len[s0 + i] = S.acc[i];
      P.emit_count[s0 + i] = S.e[i];
      if (P.status) P.status[s0 + i] = S.st[i];
      if (P.emit_offsets) P.emit_offsets[s0 + i] = S.off[i];
    }
  }
  return carry + total;
}

// Loads of one tile, issued together by the loading lanes: the tile's slots
// (agent scope; absent slots read 0), its drafts and budgets.
struct TileLoads {
  uint64_t v[kKPL];
  int d[kKPL];
  int rem;
};

__device__ inline void issue_tile(const GreedyParams &P, int s0, int ns, TileLoads &L) {
  const int t = threadIdx.x, kp1 = P.k + 1, nk = ns * kp1 * P.chunks, nd = ns * P.k;
  const uint64_t *slot0 = P.keys + static_cast<size_t>(s0) * kp1 * P.chunks;
#pragma unroll
  for (int i = 0; i < kKPL; ++i) {
    const int f = t + i * kLoadLanes;
    L.v[i] = f < nk ? load_agent(slot0 + f) : kEmptyKey;
    L.d[i] = f < nd ? P.draft[static_cast<size_t>(s0) * P.k + f] : 0;
  }
  L.rem = (t < ns && P.remaining) ? P.remaining[s0 + t] : -1;
}

constexpr int kMaxPolls = 1 << 22;   // about 4 s of polling: a bound every wait reaches

// Workgroup 0 of the single-launch verify.
__device__ void finish_verify(const GreedyParams &P) {
  __shared__ TileShared S;
  const int t = threadIdx.x, kp1 = P.k + 1;
  const bool loader = t < kLoadLanes;
  const int per = tile_sequences(P.k, P.chunks);
  int carry = 0, polls = 0;
  bool timed_out = false;
  TileLoads L;
#pragma unroll
  for (int i = 0; i < kKPL; ++i) L.v[i] = kEmptyKey;
  if (loader) issue_tile(P, 0, min(per, P.B), L);
  for (int s0 = 0; s0 < P.B; s0 += per) {
    const int ns = min(per, P.B - s0), nk = ns * kp1 * P.chunks;
    const uint64_t *slot0 = P.keys + static_cast<size_t>(s0) * kp1 * P.chunks;
    // wait until every slot of the tile is published (re-reading only the
    // missing ones); the bound keeps the wait finite
    while (true) {
      bool present = true;
#pragma unroll
      for (int i = 0; i < kKPL; ++i) present = present && L.v[i] != 0ull;
      if (__syncthreads_and(present)) break;
      if (++polls >= kMaxPolls) { timed_out = true; break; }
      __builtin_amdgcn_s_sleep(1);
      if (loader) {
#pragma unroll
        for (int i = 0; i < kKPL; ++i) {
          const int f = t + i * kLoadLanes;
          if (L.v[i] == 0ull) L.v[i] = load_agent(slot0 + f);
        }
      }
    }
    if (loader) {
#pragma unroll
      for (int i = 0; i < kKPL; ++i) {
        const int f = t + i * kLoadLanes;
        if (f < nk) S.key[f] = L.v[i];
        if (f < ns * P.k) S.d[f] = L.d[i];
      }
      if (t < ns) {
        S.rem[t] = L.rem;
        S.stop[t] = P.k;
        S.st[t] = timed_out ? SPEC_ST_INCOMPLETE : 0;
      }
    }
    __syncthreads();
    // the next tile's loads are in flight while this one is committed
    if (loader && s0 + per < P.B) issue_tile(P, s0 + per, min(per, P.B - s0 - per), L);
    carry = commit_tile(P, S, s0, ns, carry);
  }
  if (P.emit_offsets && t == kLoadLanes) P.emit_offsets[P.B] = carry;
  // every slot back to 0 for the next call (ordered before it by the launch)
  for (int f = t; f < P.nprod; f += kThreads) P.keys[f] = 0ull;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void greedy_verify_kernel(GreedyParams P) {
  if (blockIdx.x == 0) finish_verify(P);
  else stream_chunk<BF16, true>(P, static_cast<int>(blockIdx.x) - 1);
}

// ------------------------------------------------ tree, single launch ----
// The same single launch for candidate trees (N = k + 1 nodes per sequence):
// workgroup 0 polls a tile of sequences' chunk keys as finish_verify does,
// then commits the tile in LDS with the rule of tree_commit_kernel (one lane
// per node folds its row and finds the child that proposed the row's
// argmax, one lane per sequence walks from the root).  Used when one whole
// tree's chunk keys fit a tile.
struct TreeTileShared {
  uint64_t key[kTileKeys];   // the tile's chunk keys, node-major
  int d[kTileKeys];          // drafts; after the walk: emitted tokens
  int fc[kTileKeys];         // first child; after the walk: path nodes
  int ns[kTileKeys];         // next sibling
  int tok[kTileKeys];        // argmax of each node's row
  int nxt[kTileKeys];        // child proposing that argmax, or -1
  int st[kTileSeq];          // status bits
  int cnt[kTileSeq];         // budgets, then emit counts
  int scan[kThreads / kWave + 1];
};

__host__ __device__ inline int tree_tile_sequences(int N, int chunks) {
  return min(kTileSeq, (kTileKeys / chunks) / N);
}

__device__ void finish_tree(const GreedyParams &P) {
  __shared__ TreeTileShared S;
  const int t = threadIdx.x, N = P.k + 1;
  const bool loader = t < kLoadLanes;
  const int per = tree_tile_sequences(N, P.chunks);
  int carry = 0, polls = 0;
  bool timed_out = false;
  uint64_t v[kKPL];
  for (int s0 = 0; s0 < P.B; s0 += per) {
    const int nseq = min(per, P.B - s0), nrows = nseq * N, nk = nrows * P.chunks;
    const uint64_t *slot0 = P.keys + static_cast<size_t>(s0) * N * P.chunks;
    const size_t r0 = static_cast<size_t>(s0) * N;
    // the tile's slots, drafts, links and budgets, issued together
#pragma unroll
    for (int i = 0; i < kKPL; ++i) {
      const int f = t + i * kLoadLanes;
      v[i] = loader && f < nk ? load_agent(slot0 + f) : kEmptyKey;
    }
    for (int r = t; r < nrows; r += kThreads) {
      S.d[r] = P.draft[r0 + r];
      S.fc[r] = P.first_child[r0 + r];
      S.ns[r] = P.next_sibling[r0 + r];
    }
    if (t < nseq) {
      S.st[t] = 0;
      S.cnt[t] = P.remaining ? P.remaining[s0 + t] : -1;
    }
    // wait until every slot of the tile is published (re-reading only the
    // missing ones); the bound keeps the wait finite
    while (true) {
      bool present = true;
#pragma unroll
      for (int i = 0; i < kKPL; ++i) present = present && v[i] != 0ull;
      if (__syncthreads_and(present)) break;
      if (++polls >= kMaxPolls) { timed_out = true; break; }
      __builtin_amdgcn_s_sleep(1);
      if (loader) {
#pragma unroll
        for (int i = 0; i < kKPL; ++i) {
          const int f = t + i * kLoadLanes;
          if (v[i] == 0ull) v[i] = load_agent(slot0 + f);
        }
      }
    }
    if (loader) {
#pragma unroll
      for (int i = 0; i < kKPL; ++i) {
        const int f = t + i * kLoadLanes;
        if (f < nk) S.key[f] = v[i];
      }
    }
    __syncthreads();
    // one lane per node: fold its row's chunk keys; check its draft and links
    for (int r = t; r < nrows; r += kThreads) {
      const uint64_t *kr = S.key + r * P.chunks;
      uint64_t best = 0ull;
      for (int c = 0; c < P.chunks; ++c) best = kr[c] > best ? kr[c] : best;
      S.tok[r] = argmax_key_index(best);
      const int seq = r / N, node = r - seq * N;
      const int d = S.d[r], fc = S.fc[r], ns = S.ns[r];
      int bits = timed_out ? SPEC_ST_INCOMPLETE : 0;
      if (node > 0 && (d < 0 || d >= P.V)) bits |= SPEC_ST_DRAFT_OOR;
      if ((fc != -1 && (fc <= node || fc >= N)) || (ns != -1 && (ns <= node || ns >= N)))
        bits |= SPEC_ST_BAD_STATE;
      if (bits) atomicOr(&S.st[seq], bits);
    }
    __syncthreads();
    // the child proposing each node's argmax (only in trees whose every link
    // points forward, so each walk ends)
    for (int r = t; r < nrows; r += kThreads) {
      const int seq = r / N, base = seq * N;
      int c = -1;
      if (!(S.st[seq] & SPEC_ST_BAD_STATE)) {
        c = S.fc[r];
        while (c != -1 && S.d[base + c] != S.tok[r]) c = S.ns[base + c];
      }
      S.nxt[r] = c;
    }
    __syncthreads();
    // one lane per sequence: the walk from the root
    int cnt = 0;
    if (t < nseq) {
      const int b = s0 + t, sb = t * N;
      const int st = S.st[t], rem = S.cnt[t];
      int acc = 0;
      if (!(st & SPEC_ST_BAD_STATE) && rem != 0) {
        int cur = 0;
        while (true) {
          const int tk = S.tok[sb + cur];
          const int c = S.nxt[sb + cur];
          S.d[sb + cnt] = tk;                          // drafts and links are no longer read:
          S.fc[sb + cnt] = cur;                        // their rows now hold tokens and path
          ++cnt;
          if (c != -1) ++acc;
          if ((P.eos >= 0 && tk == P.eos) || cnt == rem || c == -1) break;
          cur = c;
        }
      }
      S.cnt[t] = cnt;
      P.accept_len[b] = acc;
      P.emit_count[b] = cnt;
      if (P.status) P.status[b] = st;
    }
    __syncthreads();
    for (int r = t; r < nrows; r += kThreads) {
      const int seq = r / N, node = r - seq * N;
      const bool kept = node < S.cnt[seq];
      P.out_tokens[r0 + r] = kept ? S.d[r] : -1;
      P.path[r0 + r] = kept ? S.fc[r] : -1;
    }
    if (P.emit_offsets) {
      int total;
      const int ex = block_excl_scan(t < nseq ? cnt : 0, S.scan, &total);
      if (t < nseq) P.emit_offsets[s0 + t] = carry + ex;
      carry += total;
    }
    __syncthreads();
  }
  if (P.emit_offsets && t == 0) P.emit_offsets[P.B] = carry;
  // every slot back to 0 for the next call (ordered before it by the launch)
  for (int f = t; f < P.nprod; f += kThreads) P.keys[f] = 0ull;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void tree_verify_kernel(GreedyParams P) {
  if (blockIdx.x == 0) finish_tree(P);
  else stream_chunk<BF16, true>(P, static_cast<int>(blockIdx.x) - 1);
}



constexpr int kCommitThreads = 1024;
constexpr int kCommitRows = 1024;   // row keys folded per tile (LDS)
constexpr int kKeysPerThread = 16;  // chunk keys in flight per lane
static_assert(kCommitRows == kCommitThreads, "one row (and at most one draft) per lane of a tile");

// Two-launch path (rows with more chunk keys than a finisher tile holds): one
// workgroup.  Per tile of sequences, every global read (chunk keys, drafts,
// budgets) is issued at once into LDS; the walk then runs from LDS only.  The
// slots read are returned to 0.
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
    uint64_t *kb = P.keys + static_cast<size_t>(s0) * kp1 * P.chunks;
    const bool has_d = t < ns * P.k, has_r = t < nrows;
    const int dv = has_d ? P.draft[static_cast<size_t>(s0) * P.k + t] : 0;
    const int rv = t < ns && P.remaining ? P.remaining[s0 + t] : -1;   // negative: no budget
    uint64_t best = 0ull;
    if (has_r) {
      uint64_t *rk = kb + static_cast<size_t>(t) * P.chunks;
      for (int c0 = 0; c0 < P.chunks; c0 += kKeysPerThread) {
        uint64_t kr[kKeysPerThread];
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) kr[q] = c0 + q < P.chunks ? rk[c0 + q] : 0ull;
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) best = kr[q] > best ? kr[q] : best;
      }
      for (int c = 0; c < P.chunks; ++c) rk[c] = 0ull;   // the workspace returns to zero
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
      uint64_t *rk = P.keys + (r0 + t) * P.chunks;
      for (int c0 = 0; c0 < P.chunks; c0 += kKeysPerThread) {
        uint64_t kr[kKeysPerThread];
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) kr[q] = c0 + q < P.chunks ? rk[c0 + q] : 0ull;
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) best = kr[q] > best ? kr[q] : best;
      }
      for (int c = 0; c < P.chunks; ++c) rk[c] = 0ull;   // the workspace returns to zero
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

// Argument checks and launch of a greedy verification on the chunk-key array
// `keys` (wsb bytes).  noalloc: the keys are the library's static scratch (any
// contents on entry), so the two-launch path is taken, whose streaming kernel
// writes every slot before the commit reads it.
static int greedy_verify_launch(const void *logits, spec_dtype dt, int B, int k, int V,
                                const int32_t *draft, int32_t eos_id, const int32_t *remaining,
                                int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                                int32_t *emit_offsets, int32_t *status, void *keys, bool noalloc,
                                spec_stream_t stream) {
  const size_t elt = dt == SPEC_BF16 ? 2 : 4;
  const int chunks = greedy_chunks(V, dt);
  const long long nblocks = static_cast<long long>(B) * (k + 1) * chunks;
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
  P.keys = static_cast<uint64_t *>(keys);
  P.nprod = static_cast<int>(nblocks);
  P.first_child = P.next_sibling = nullptr;
  P.path = nullptr;
  (void)elt;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (!noalloc && tile_sequences(k, chunks) >= 1 && nblocks + 1 < INT32_MAX) {
    // one launch: workgroup 0 commits, the others stream
    const dim3 grid(static_cast<unsigned>(nblocks + 1));
    if (dt == SPEC_BF16) hipLaunchKernelGGL(greedy_verify_kernel<true>, grid, dim3(kThreads), 0, s, P);
    else hipLaunchKernelGGL(greedy_verify_kernel<false>, grid, dim3(kThreads), 0, s, P);
    return launch_status();
  }
  if (dt == SPEC_BF16)
    hipLaunchKernelGGL(greedy_chunk_kernel<true>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL(greedy_chunk_kernel<false>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  hipLaunchKernelGGL(greedy_commit_kernel, dim3(1), dim3(kCommitThreads), 0, s, P);
  return launch_status();
}

// Host checks shared by both greedy entry points; ws may be null (no-alloc).
static int greedy_verify_check(const void *logits, spec_dtype dt, int B, int k, int V, const int32_t *draft,
                               const int32_t *remaining, int32_t *accept_len, int32_t *emit_count,
                               int32_t *out_tokens, int32_t *emit_offsets, int32_t *status,
                               const void *ws, size_t *wsb_out) {
  if (!logits || !draft || !accept_len || !emit_count || !out_tokens) return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (B < 1 || k < 1 || V < 1 || V >= INT32_MAX - 1) return SPEC_EINVAL;
  if (k > SPEC_MAX_K) return SPEC_ECAPACITY;
  const size_t elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(logits, elt)) return SPEC_EINVAL;
  const int chunks = greedy_chunks(V, dt);
  const long long nblocks = static_cast<long long>(B) * (k + 1) * chunks;
  if (nblocks >= INT32_MAX) return SPEC_EINVAL;
  const size_t wsb = greedy_ws_bytes(B, k, chunks);
  *wsb_out = wsb;
  const size_t nl = static_cast<size_t>(B) * (k + 1) * V * elt;
  const void *ins[] = {logits, draft, remaining, ws};
  const size_t in_n[] = {nl, static_cast<size_t>(B) * k * 4, static_cast<size_t>(B) * 4, ws ? wsb : 0};
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
  return SPEC_OK;
}

extern "C" int spec_verify_greedy(const void *logits, spec_dtype dt, int B, int k, int V,
                                  const int32_t *draft, int32_t eos_id, const int32_t *remaining,
                                  int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                                  int32_t *emit_offsets, int32_t *status, void *ws,
                                  size_t ws_bytes, spec_stream_t stream) {
  if (!ws) return SPEC_EINVAL;
  size_t wsb = 0;
  const int rc = greedy_verify_check(logits, dt, B, k, V, draft, remaining, accept_len, emit_count, out_tokens,
                                     emit_offsets, status, ws, &wsb);
  if (rc != SPEC_OK) return rc;
  if (ws_bytes < wsb || !aligned(ws, 256)) return SPEC_EWORKSPACE;
  return greedy_verify_launch(logits, dt, B, k, V, draft, eos_id, remaining, accept_len, emit_count, out_tokens,
                              emit_offsets, status, ws, false, stream);
}

// ----------------------------------------------------------- no-alloc ----
// Chunk keys of spec_verify_greedy_noalloc: a static array on every device the
// library runs on (kept until the process ends).  Host code never passes the
// array's name to a kernel or a copy: the name is a host-side stand-in, not a
// device address.  The device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
static __device__ __align__(256) uint64_t scratch[SPEC_GREEDY_SCRATCH_BYTES / sizeof(uint64_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SPEC_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}
}  // namespace

extern "C" int spec_verify_greedy_noalloc(const void *logits, spec_dtype dt, int B, int k, int V,
                                          const int32_t *draft, int32_t eos_id, const int32_t *remaining,
                                          int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                                          int32_t *emit_offsets, int32_t *status, spec_stream_t stream) {
  size_t wsb = 0;
  int rc = greedy_verify_check(logits, dt, B, k, V, draft, remaining, accept_len, emit_count, out_tokens,
                               emit_offsets, status, nullptr, &wsb);
  if (rc != SPEC_OK) return rc;
  if (wsb > SPEC_GREEDY_SCRATCH_BYTES) return SPEC_ECAPACITY;
  void *keys = nullptr;
  rc = scratch_address(&keys);
  if (rc != SPEC_OK) return rc;
  return greedy_verify_launch(logits, dt, B, k, V, draft, eos_id, remaining, accept_len, emit_count, out_tokens,
                              emit_offsets, status, keys, true, stream);
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
  P.nprod = static_cast<int>(nblocks);
  P.first_child = first_child;
  P.next_sibling = next_sibling;
  P.path = path;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (tree_tile_sequences(N, chunks) >= 1 && nblocks + 1 < INT32_MAX) {
    // one launch: workgroup 0 commits tiles of trees while the rest stream
    const dim3 g(static_cast<unsigned>(nblocks + 1));
    if (dt == SPEC_BF16)
      hipLaunchKernelGGL(tree_verify_kernel<true>, g, dim3(kThreads), 0, s, P);
    else
      hipLaunchKernelGGL(tree_verify_kernel<false>, g, dim3(kThreads), 0, s, P);
    return launch_status();
  }
  if (dt == SPEC_BF16)
    hipLaunchKernelGGL(greedy_chunk_kernel<true>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL(greedy_chunk_kernel<false>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  hipLaunchKernelGGL(tree_commit_kernel, dim3(1), dim3(kCommitThreads), 0, s, P);
  return launch_status();
}
