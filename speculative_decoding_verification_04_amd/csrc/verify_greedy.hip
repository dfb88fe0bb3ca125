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
//     Each wave's maximum comes from plain max instructions and DPP lane
//     moves; only the lanes holding it search their own elements for its
//     first index (a DPP minimum picks the lowest), and the waves' 64-bit
//     keys meet in LDS (value order high, UINT32_MAX - index low; the largest
//     key is the argmax at the lowest index).  The chunk's key is published
//     with one agent-scope store into its workspace slot.  A published key is
//     never 0 (an empty chunk publishes 1), so a slot is its own flag.
//   * workgroup 0, the finisher, takes the batch in tiles of sequences whose
//     slots are laid out in its polling order.  Each lane polls its own few
//     slots with agent-scope loads (no workgroup barrier between polls, only
//     missing slots re-read), folds what arrived per row in registers and
//     into the row's maximum in LDS, and returns each arrived slot to 0 (the
//     workspace stays zero-filled between calls).  The lane that completes a
//     row tests its stop conditions (mismatch, EOS) with an LDS minimum per
//     sequence.  After the tile's last arrival wave 0 applies the budgets,
//     counts the accepted drafts and scans the emit counts, and the rows
//     write their tokens.
// Producers never wait: the finisher is one workgroup whose wait ends when
// every producer has published, and producers depend on nothing.  Device-
// scope atomics on shared counters are avoided altogether (on a multi-XCD
// part they serialise per address).  Sequences whose rows need more chunk
// keys than one finisher tile holds fall back to two launches: the streaming
// kernel, then a one-workgroup commit (tree verification uses the same
// streaming kernel with its own commit).
#include "common.h"

#include <algorithm>
#include <atomic>
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
  uint64_t *keys;     // chunk-key slots; zero between calls (the slot flags)
  int nprod;          // producer workgroups of the single-launch path
  int tile_seq;       // linear single launch: sequences per finisher tile (slots
                      // in the tile's polling order); 0: slot row * chunks + c
  int tile_span;      // slots per full tile in that order
  int max_polls;      // the single-launch finishers' wait bound (polls)
  // tree verification only (k + 1 = N nodes per sequence)
  const int32_t *first_child, *next_sibling;
  int32_t *path;
};

// Finisher tiles of the linear single launch.  The finisher's lanes poll a
// tile's chunk-key slots kSlotsPerLane at a time per lane, in phases of
// kPhaseSlots slots; a tile holds at most kArrRows rows and kArrSlots slots.
constexpr int kSlotsPerLane = 4;                        // few enough that nothing spills to scratch
constexpr int kPhaseSlots = kThreads * kSlotsPerLane;   // chunk keys polled at once
constexpr int kArrSlots = 8 * kPhaseSlots;              // chunk keys per tile
constexpr int kArrRows = 1024;                          // rows per tile
constexpr int kTileSeq = 256;                           // sequences per tile (both finishers)

__host__ __device__ inline int tile_sequences(int k, int chunks) {
  const int rows = min(kArrRows, kArrSlots / chunks);
  return min(kTileSeq, rows / (k + 1));
}

// Slots per lane n and lanes L of a phase of m slots: as many slots per lane
// as keep L >= 16 (a lane's slots then sit in different 128-byte lines), at
// most kSlotsPerLane.
__host__ __device__ inline void phase_shape(int m, int &n, int &L) {
  n = max(1, min(kSlotsPerLane, m / 16));
  L = (m + n - 1) / n;
}

// Where logical slot f (0 <= f < nk; row-major over the tile's rows and
// chunks) of a tile of nk slots is stored.  In a phase of m slots, lane t
// polls the n consecutive logical slots n*t .. n*t+n-1 (chunks of one or two
// rows, so they fold in registers), stored at positions i*L + t: each of a
// lane's loads reaches a different cache line and one load instruction of a
// wave reads consecutive positions.  Several loads of one line by one lane
// were measured to wait on each other (2 us more per call on small batches).
// A phase takes n*L <= m + 3 positions.
__host__ __device__ inline int slot_position(int f, int nk) {
  const int ph = f / kPhaseSlots, w = f - ph * kPhaseSlots;
  int n, L;
  phase_shape(min(kPhaseSlots, nk - ph * kPhaseSlots), n, L);
  return ph * kPhaseSlots + (w % n) * L + w / n;
}

// Positions between the starts of consecutive tiles (a full tile's slots and
// the last phase's padding).
inline size_t tile_span(int k, int chunks) {
  return round_up(static_cast<size_t>(tile_sequences(k, chunks)) * (k + 1) * chunks + 3, 4);
}

// Slots of the row-major layout (two-launch path): B*(k+1)*chunks.
inline size_t greedy_plain_bytes(int B, int k, int chunks) {
  return round_up(static_cast<size_t>(B) * (k + 1) * chunks * sizeof(uint64_t), 256);
}

// Slots of either layout: whole tiles in polling order, or row-major.
inline size_t greedy_ws_bytes(int B, int k, int chunks) {
  const int per = tile_sequences(k, chunks);
  size_t b = greedy_plain_bytes(B, k, chunks);
  if (per >= 1)
    b = std::max(b, round_up(static_cast<size_t>((B + per - 1) / per) * tile_span(k, chunks) * sizeof(uint64_t), 256));
  return b;
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
  __shared__ uint64_t sh_key[kWaves];

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
  // the lane holds no element at all), then each wave's maximum through DPP.
  float lmax = fmaxf(hv, tv);
#pragma unroll
  for (int u = 0; u < U; ++u) lmax = fmaxf(lmax, vec_max<BF16>(buf[u]));
  const float wm = wave_max_dpp(lmax);

  // Only lanes holding their wave's maximum look for its first index among
  // their own elements, visited in increasing index order (head, vectors
  // u = 0..U-1, tail); a DPP minimum gives the wave's first index and one
  // 64-bit key per wave goes to LDS.  The largest of the waves' keys is the
  // chunk's (larger value first, then the lower index).
  int cand = INT_MAX;
  if (lmax == wm) {
    if (has_tail && tv == wm) cand = s + nv * VEC + t;
#pragma unroll
    for (int u = U - 1; u >= 0; --u) {
      const int vi = t + u * kThreads;
      const int q = vec_find<BF16>(buf[u], wm);
      if (vi < nv && q < VEC) cand = s + vi * VEC + q;
    }
    if (has_head && hv == wm) cand = t;
  }
  cand = wave_min(cand);
  if (lane == 0) sh_key[w] = cand == INT_MAX ? kEmptyKey : argmax_key(wm, cand);
  __syncthreads();
  if (t == 0) {
    uint64_t key = sh_key[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) key = sh_key[i] > key ? sh_key[i] : key;
    size_t pos = static_cast<size_t>(row) * P.chunks + c;
    if (PUBLISH && P.tile_seq > 0) {
      // the linear finisher's polling order: tile q, then slot_position
      const int kp1 = P.k + 1, q = row / kp1 / P.tile_seq, s0 = q * P.tile_seq;
      const int nk = min(P.tile_seq, P.B - s0) * kp1 * P.chunks;
      pos = static_cast<size_t>(q) * P.tile_span + slot_position((row - s0 * kp1) * P.chunks + c, nk);
    }
    uint64_t *slot = P.keys + pos;
    if constexpr (PUBLISH) __hip_atomic_store(slot, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *slot = key;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void greedy_chunk_kernel(GreedyParams P) {
  stream_chunk<BF16, false>(P, blockIdx.x);
}

// ---------------------------------------------------------------- commit ----
// Slot polling shared by the finishers: a tile's chunk-key slots are read
// with agent-scope loads (absent slots read 0) and re-read until present.
constexpr int kTileKeys = 1024;     // chunk keys per tile of the tree finisher
constexpr int kLoadLanes = kThreads - kWave;                              // waves 0 .. kWaves-2
constexpr int kKPL = (kTileKeys + kLoadLanes - 1) / kLoadLanes;           // slots per loading lane
static_assert(kTileSeq <= kLoadLanes, "one loading lane per sequence of a tile");
constexpr int kMaxPolls = 1 << 22;   // about 4 s of polling: the default bound every wait reaches
constexpr int kWaitVm0 = 0x0F70;     // s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt not waited for

// The linear finisher folds results as they arrive.  Every lane polls its own
// few consecutive slots of the tile at a time (all in flight, no workgroup
// barrier between polls; a tile of more slots than the lanes hold is polled in
// phases, in the producers' order), folds the arrived keys of each row in
// registers and then into the row's maximum in LDS.  The lane whose keys
// complete a row decides that row (argmax, mismatch, EOS).  After the tile's
// last arrival wave 0 commits the sequences (counts, offsets) and the tokens
// are written.
struct ArrivalShared {
  unsigned long long best[kArrRows];   // running maximum key of each row
  int cnt[kArrRows];                   // chunk keys seen per row
  int tok[kArrRows];                   // argmax of each decided row
  int d[kArrRows];                     // the tile's drafts (ns * k < rows)
  int stop[kTileSeq];                  // first row that stops the sequence (LDS minimum)
  int rem[kTileSeq];                   // budgets
  int st[kTileSeq];                    // status bits
  int e[kTileSeq];                     // emit counts
  int timed_out;
};

// Row r (row j of the tile's sequence b) has its argmax key `best`: record
// the argmax and test the row's stop conditions (draft j < k: a mismatch or
// EOS stops after emitting row j).
__device__ inline void decide_row(const GreedyParams &P, ArrivalShared &S, int r, int b, int j, uint64_t best) {
  const int tok = argmax_key_index(best);
  S.tok[r] = tok;
  if (j < P.k) {
    const int d = S.d[b * P.k + j];
    if (d < 0 || d >= P.V) atomicOr(&S.st[b], SPEC_ST_DRAFT_OOR);
    if (tok != d || (P.eos >= 0 && tok == P.eos)) atomicMin(&S.stop[b], j);
  }
}

// n chunk keys of row r (row j of sequence b) arrived, their maximum is m.
// The count is an acquire-release LDS increment: the lane that completes the
// row sees every other lane's maximum of that row.
__device__ inline void arrive(const GreedyParams &P, ArrivalShared &S, int r, int b, int j, uint64_t m, int n) {
  atomicMax(&S.best[r], static_cast<unsigned long long>(m));
  if (__hip_atomic_fetch_add(&S.cnt[r], n, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) + n == P.chunks)
    decide_row(P, S, r, b, j, atomicMax(&S.best[r], 0ull));   // the row's maximum, every key folded in
}

// The tile of sequences starting at s0: its first slot.
__device__ inline uint64_t *tile_slots(const GreedyParams &P, int s0) {
  return P.keys + static_cast<size_t>(s0 / P.tile_seq) * P.tile_span;
}

// Polls of this lane's slots (bit i of mask: logical slot ph*kPhaseSlots +
// n*t + i, at position ph*kPhaseSlots + i*L + t) of phase ph of a tile.
__device__ inline void poll_slots(const uint64_t *slot0, int ph, int L, unsigned mask, uint64_t *v) {
  const uint64_t *p = slot0 + ph * kPhaseSlots + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kSlotsPerLane; ++i)
    if ((mask >> i) & 1u) v[i] = load_agent(p + i * L);
}

// The slots lane t holds in phase ph of a tile of nk slots (n per lane), as a
// bit mask.
__device__ inline unsigned lane_slots(int ph, int nk, int n) {
  const int f0 = ph * kPhaseSlots + threadIdx.x * n;
  unsigned m = 0u;
#pragma unroll
  for (int i = 0; i < kSlotsPerLane; ++i)
    if (i < n && f0 + i < nk) m |= 1u << i;
  return m;
}

// Loads of one tile's slots (phase 0), drafts and budgets into registers.
__device__ inline void issue_arrivals(const GreedyParams &P, int s0, int ns, uint64_t *v, int *dv, int &rv) {
  const int t = threadIdx.x, kp1 = P.k + 1, nk = ns * kp1 * P.chunks, nd = ns * P.k;
#pragma unroll
  for (int i = 0; i < kSlotsPerLane; ++i) v[i] = 0ull;
  int n, L;
  phase_shape(min(kPhaseSlots, nk), n, L);
  poll_slots(tile_slots(P, s0), 0, L, lane_slots(0, nk, n), v);
#pragma unroll
  for (int i = 0; i < kArrRows / kThreads; ++i) {
    const int f = t + i * kThreads;
    dv[i] = f < nd ? P.draft[static_cast<size_t>(s0) * P.k + f] : 0;
  }
  rv = (t < ns && P.remaining) ? P.remaining[s0 + t] : -1;
}

// Workgroup 0 of the single-launch verify.
__device__ void finish_verify(const GreedyParams &P) {
  __shared__ ArrivalShared S;
  const int t = threadIdx.x, lane = t & (kWave - 1), kp1 = P.k + 1;
  const int per = tile_sequences(P.k, P.chunks);
  int carry = 0, polls = 0;
  uint64_t v[kSlotsPerLane];
  int dv[kArrRows / kThreads];
  int rv;
  if (t == 0) S.timed_out = 0;
  issue_arrivals(P, 0, min(per, P.B), v, dv, rv);
  for (int s0 = 0; s0 < P.B; s0 += per) {
    const int ns = min(per, P.B - s0), nrows = ns * kp1, nk = nrows * P.chunks;
    uint64_t *slot0 = tile_slots(P, s0);
    // the tile's LDS state
    for (int r = t; r < nrows; r += kThreads) {
      S.best[r] = 0ull;
      S.cnt[r] = 0;
    }
#pragma unroll
    for (int i = 0; i < kArrRows / kThreads; ++i) {
      const int f = t + i * kThreads;
      if (f < ns * P.k) S.d[f] = dv[i];
    }
    if (t < ns) {
      S.stop[t] = P.k;
      S.rem[t] = rv;
      S.st[t] = 0;
    }
    __syncthreads();
    // poll this lane's slots until each has arrived, phase after phase; the
    // bound keeps the wait finite (and a timeout anywhere ends every lane's wait)
    for (int ph = 0; ph * kPhaseSlots < nk; ++ph) {
      int n, L;                                               // slots per lane, lanes
      phase_shape(min(kPhaseSlots, nk - ph * kPhaseSlots), n, L);
      const int f0 = ph * kPhaseSlots + t * n;                // this lane's first logical slot of the phase
      uint64_t *pos0 = slot0 + ph * kPhaseSlots + t;          // logical slot f0 + i is at pos0[i * L]
      unsigned miss = lane_slots(ph, nk, n);
      if (ph > 0) poll_slots(slot0, ph, L, miss, v);
      const int r_lo = f0 / P.chunks, r_hi = (f0 + n - 1) / P.chunks;
      const int b_lo = r_lo / kp1, j_lo = r_lo - b_lo * kp1;   // row r_lo is row j_lo of sequence b_lo
      unsigned filled = 0u;                                     // slots counted as empty after a timeout
      while (true) {
        unsigned got = 0u;
#pragma unroll
        for (int i = 0; i < kSlotsPerLane; ++i)
          if (((miss >> i) & 1u) && v[i] != 0ull) got |= 1u << i;
        miss &= ~got;
        // the arrivals are folded per row in registers first (a lane's slots
        // are consecutive, so they span few rows), then once per row into LDS
        for (int r = r_lo, b = b_lo, j = j_lo; got != 0u && r <= r_hi; ++r) {
          const int lo = max(r * P.chunks - f0, 0), hi = min(n, (r + 1) * P.chunks - f0);
          const unsigned g = got & ((1u << hi) - 1u) & ~((1u << lo) - 1u);   // row r's slots among them
          const int rb = b, rj = j;
          if (++j == kp1) {
            j = 0;
            ++b;
          }
          if (g == 0u) continue;
          got &= ~g;
          if (g & filled) atomicOr(&S.st[rb], SPEC_ST_INCOMPLETE);
          uint64_t m = 0ull;
#pragma unroll
          for (int i = 0; i < kSlotsPerLane; ++i) {
            if ((g >> i) & 1u) {
              m = v[i] > m ? v[i] : m;
              pos0[i * L] = 0ull;       // the workspace returns to zero (seen by the next launch)
            }
          }
          arrive(P, S, r, rb, rj, m, __builtin_popcount(g));
        }
        if (miss == 0u) break;
        if (__hip_atomic_load(&S.timed_out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) || ++polls >= P.max_polls) {
          // the wait is over: the slots still missing count as empty chunks
          // and their sequences are marked incomplete
          __hip_atomic_store(&S.timed_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
          for (int i = 0; i < kSlotsPerLane; ++i)
            if ((miss >> i) & 1u) v[i] = kEmptyKey;
          filled = miss;
          continue;
        }
        // this lane's stores (zeroed slots, outputs) complete before its next
        // polls are issued, about 0.2 us apart (both measured faster than
        // letting polls overtake the stores or polling back to back)
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_s_sleep(8);
        poll_slots(slot0, ph, L, miss, v);
      }
    }
    // the next tile's loads go out before the wait for the other lanes
    if (s0 + per < P.B) issue_arrivals(P, s0 + per, min(per, P.B - s0 - per), v, dv, rv);
    __syncthreads();
    // wave 0 commits the tile's sequences, 64 at a time: emitted count
    // (first stop row + 1, capped by the budget), accepted drafts (every
    // emitted row before the last matched; the last emitted row counts if it
    // matched its draft), the emit offsets after the carry
    if (t < kWave) {
      for (int base = 0; base < ns; base += kWave) {
        const int b = base + lane;
        int cnt = 0;
        if (b < ns) {
          const int rem = S.rem[b];
          cnt = S.stop[b] + 1;
          if (rem >= 0) cnt = min(cnt, rem);
          int acc = 0;
          if (cnt > 0) {
            const int last = cnt - 1;
            acc = last + ((last < P.k && S.tok[b * kp1 + last] == S.d[b * P.k + last]) ? 1 : 0);
          }
          S.e[b] = cnt;
          P.accept_len[s0 + b] = acc;
          P.emit_count[s0 + b] = cnt;
          if (P.status) P.status[s0 + b] = S.st[b];
        }
        const int inc = wave_incl_scan(cnt);
        if (P.emit_offsets && b < ns) P.emit_offsets[s0 + b] = carry + inc - cnt;
        carry += read_lane(inc, kWave - 1);
      }
    }
    __syncthreads();
    // the emitted tokens, one lane per row
    int32_t *out = P.out_tokens + static_cast<size_t>(s0) * kp1;
    for (int r = t; r < nrows; r += kThreads) out[r] = r % kp1 < S.e[r / kp1] ? S.tok[r] : -1;
    if (s0 + per < P.B) __syncthreads();   // the next tile's LDS state overwrites this one's
  }
  if (P.emit_offsets && t == 0) P.emit_offsets[P.B] = carry;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void greedy_verify_kernel(GreedyParams P) {
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
      if (++polls >= P.max_polls) { timed_out = true; break; }
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

// Wait bound of the single-launch finishers (0: the default).
static std::atomic<int> g_wait_bound{0};

static int wait_bound() {
  const int b = g_wait_bound.load(std::memory_order_relaxed);
  return b > 0 ? b : kMaxPolls;
}

extern "C" int spec_set_wait_bound(int polls) {
  return g_wait_bound.exchange(polls > 0 ? polls : 0, std::memory_order_relaxed);
}

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
  P.tile_seq = 0;
  P.tile_span = 0;
  P.max_polls = wait_bound();
  (void)elt;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (!noalloc && tile_sequences(k, chunks) >= 1 && nblocks + 1 < INT32_MAX) {
    P.tile_seq = tile_sequences(k, chunks);
    P.tile_span = static_cast<int>(tile_span(k, chunks));
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
  // the two-launch path keeps its chunk keys row-major
  if (greedy_plain_bytes(B, k, greedy_chunks(V, dt)) > SPEC_GREEDY_SCRATCH_BYTES) return SPEC_ECAPACITY;
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
  P.tile_seq = 0;
  P.tile_span = 0;
  P.max_polls = wait_bound();
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
