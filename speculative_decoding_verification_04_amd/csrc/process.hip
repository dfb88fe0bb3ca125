// Row statistics of processed sampling distributions (temperature, top-k,
// top-p) and their optional materialisation (gfx950).
//
// Definitions: process.h (after the zero-to-sglang walkthrough 5.1, which
// requires the processed probabilities to be the ones verified).
//
// Design.  Rows are first cut into slices of 16 KB (16384 bf16 or 8192 f32
// logits), one 256-lane workgroup each, holding the slice's raw 16-byte
// vectors in registers and working on float values (a shift or mask per bf16
// entry, three-operand maxima); a statistics workgroup per row then finishes.
//   * Top-k (K <= 256): proc_slice_kernel cuts each slice at the K-th largest
//     of its 256 lane maxima (found bit by bit with wave ballots) and lists the
//     entries at or above that cut: the vectors whose maximum reaches the cut
//     (about K) are staged in LDS and filtered by the whole workgroup.  The
//     union of the lists holds every logit at or above the row's K-th
//     largest.  Each slice also reports its ceil(K / S)-th largest lane
//     maximum; the smallest of those over the S slices is another lower bound
//     of the row's K-th largest, usually much tighter than the largest cut, so
//     the statistics see about 2K candidates instead of about K per slice.
//     When every list fits one wave, wave 0 of the statistics workgroup
//     gathers them in a single round of loads and runs every radix level on
//     them alone, with no workgroup barrier.
//   * No top-k: slice maxima (proc_slrange_kernel, or with top-p the slice
//     kernel cut at the 128th lane maximum), then the exact fixed-point weight
//     and smallest key of every slice (proc_slmass_kernel).  Temperature
//     alone keeps everything, so those sums are the result (one wave combines
//     them); with top-p the statistics kernel runs the top-p levels on the
//     union when the union carries at least top_p of the row's weight
//     (checked exactly).
// Rows whose lists overflow, and top-k beyond 256, take the whole-row path of
// the statistics kernel:
//   1. One pass over the row takes its maximum and, with top-k, a histogram of
//      the top 8 bits of the order keys.  Without top-k but with top-p, a
//      second pass takes the same histogram of counts and fixed-point weights
//      (2^-40 units, truncated).  The bucket holding the K-th largest key (or
//      the top-p boundary) is read off the histogram.
//   2. Every logit in that bucket or above is copied into LDS (it fits when at
//      most 32768 logits qualify, which covers top-k up to that size and any
//      top-p boundary whose bucket and everything above hold that few); the
//      remaining radix levels (8 bits each: 2 in all for bf16 keys, 4 for f32)
//      and the kept weight then run on that list.  Otherwise they re-read the
//      row (from L2).
//   3. The kept weight is an exact integer sum of the fixed-point weights, so
//      the result does not depend on the order logits are visited in, nor on
//      the path taken.
// Whole-row histograms are kept per lane index: bucket b, column l (256 x 64
// packed 64-bit words, 128 KB of LDS), so the 64 lanes of an atomic add hit 64
// different words.  Logits cluster in a few buckets of the top digit; one
// shared histogram serialised those adds.  A lane column receives up to about
// V/64 logits of the row.  A count-only histogram (top-k) keeps a plain count
// per word.  A histogram of counts and weights packs a count (top 10 bits) and
// a weight (low 54 bits) into one word only while no column can receive more
// than 1023 logits (V below about 57000); larger rows take two passes, one of
// counts and one of weights (at most V/64 weights of at most 2^40 units each,
// below 2^54).  Columns are summed per bucket afterwards.  The bucket scans
// are parallel suffix sums.
// Every selection keeps all logits at or above one threshold, so ties at a
// boundary are kept, as the definitions require.
#include "sample_src.h"

namespace specv {
namespace {

constexpr int kProcThreads = 1024;
constexpr int kProcWaves = kProcThreads / kWave;
constexpr int kProcU = 4;                      // 16-byte loads in flight per lane
constexpr double kFixScale = 1099511627776.0;  // 2^40 fixed-point units per unit weight
constexpr int kCntShift = 54;                   // packed histogram word: count << 54 | weight
constexpr unsigned long long kMassMask = (1ull << kCntShift) - 1;
constexpr int kPackedMaxColumn = (1 << (64 - kCntShift)) - 1;   // logits a packed column may receive
// What a whole-row histogram word holds.
enum HistMode { kHistPacked, kHistCount, kHistMass };
constexpr int kSliceThreads = 256;              // top-k slice kernel
constexpr int kSliceLoads = 8;                  // 16-byte loads per lane: one slice
constexpr int kSliceMaxS = (SPEC_PROC_MAX_V + kSliceThreads * kSliceLoads * 4 - 1) / (kSliceThreads * kSliceLoads * 4);
constexpr int kCandCap = 256 * 64 * 2;          // candidate logits that fit in the statistics kernel's LDS
// Top-p without top-k: each slice lists its entries at or above its 128th
// largest lane maximum (about 1% of the slice for Gaussian logits).  The
// statistics kernel uses the union when it carries at least top_p of the row's
// weight, which it checks exactly; else it reads the row.
constexpr int kToppRank = 128;
constexpr int kWaveList = 2048;                 // lists up to this length are finished by one wave
constexpr int kGatherS = 24;                    // wave 0 gathers the top-k lists of up to this many slices

struct ProcParams {
  const void *za, *zb;   // rows [0, rows_a) come from za, the rest from zb
  int rows_a, rows, V;
  ProcConfig cfg;
  ProcStats *stats;      // [rows]
  float *probs;          // [rows, V] or null
  // top-k candidate lists from the slice kernel (null: read the whole row)
  float *lists;          // [rows][kCandCap]: per slice, a segment of seg_cap
  int *list_cnt;         // [rows][S]: entries per segment (more than seg_cap: overflow)
  uint32_t *list_cut;    // [rows][S]: each slice listed every entry with a key at or above
  int S, seg_cap;        // slices per row, entries per segment
  int cut_rank;          // the slice kernel's cut: the cut_rank-th largest lane maximum
  uint32_t *list_lb;     // [rows][S] or null: each slice's lb_rank-th largest lane maximum
  int32_t *list_idx;     // [rows][kCandCap] or null: each listed entry's index in its row
  unsigned long long *row_pub;   // [rows][3] or null: each row's statistics as published words
                                 // (the slice kernel clears them, so they may hold anything on entry)
  int lb_rank;           // ceil(K / S): at least K logits of the row are at or above the smallest
  // rows without top-k: per slice, the key range and the fixed-point weight
  // (null: read the whole row)
  uint32_t *sl_max, *sl_min;        // [rows][S]
  unsigned long long *sl_tot;       // [rows][S]
};

template <bool BF16>
__device__ inline const void *proc_row(const ProcParams &P, int r) {
  const size_t elt = BF16 ? 2 : 4;
  if (r < P.rows_a) return static_cast<const unsigned char *>(P.za) + static_cast<size_t>(r) * P.V * elt;
  return static_cast<const unsigned char *>(P.zb) + static_cast<size_t>(r - P.rows_a) * P.V * elt;
}

// Calls f(v, z) for every entry of the row this lane owns: a scalar head up to
// the first 16-byte boundary, 16-byte vectors (kProcU per lane per step, the
// next step's loads issued before this step's entries are visited), a scalar
// tail.  The order within a lane is fixed.
template <bool BF16, int NT = kProcThreads, class F>
__device__ inline void row_foreach(const void *row, int V, F &&f) {
  constexpr int ELT = BF16 ? 2 : 4, VEC = 16 / ELT;
  constexpr int kStep = NT * kProcU;
  const int t = threadIdx.x;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row);
  const int head = min(V, static_cast<int>(((16u - (a & 15u)) & 15u) / ELT));
  const int nvec = (V - head) / VEC;
  const int tail0 = head + nvec * VEC;
  if (t < head) f(t, logit_at<BF16>(row, t));
  const uint4 *body = reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(row) + head * ELT);
  uint4 cur[kProcU], nxt[kProcU];
#pragma unroll
  for (int u = 0; u < kProcU; ++u) {
    const int i = u * NT + t;
    if (i < nvec) cur[u] = body[i];
  }
  for (int i0 = 0; i0 < nvec; i0 += kStep) {
    const bool more = i0 + kStep < nvec;
    if (more) {
#pragma unroll
      for (int u = 0; u < kProcU; ++u) {
        const int i = i0 + kStep + u * NT + t;
        if (i < nvec) nxt[u] = body[i];
      }
    }
#pragma unroll
    for (int u = 0; u < kProcU; ++u) {
      const int i = i0 + u * NT + t;
      if (i < nvec) {
        const uint32_t w[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
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
#pragma unroll
    for (int u = 0; u < kProcU; ++u) cur[u] = nxt[u];
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

// Sums the 64 columns of every bucket of the per-lane histogram into h_cnt
// (packed and count words; count words also set h_mass to 0) and h_mass
// (packed and weight words).  Contains barriers.
__device__ inline void fold_columns(const unsigned long long *lh, uint32_t *h_cnt,
                                   unsigned long long *h_mass, HistMode mode) {
  const int t = threadIdx.x;
  const int b = t >> 2, part = t & 3;          // 4 lanes per bucket, 16 columns each
  unsigned long long c = 0, m = 0;
#pragma unroll
  for (int i = 0; i < kWave / 4; ++i) {        // columns visited in a bucket-rotated order: no bank conflicts
    const unsigned long long x = lh[b * kWave + part * (kWave / 4) + ((i + b) & (kWave / 4 - 1))];
    c += mode == kHistPacked ? x >> kCntShift : (mode == kHistCount ? x : 0ull);
    m += mode == kHistPacked ? x & kMassMask : (mode == kHistMass ? x : 0ull);
  }
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    c += __shfl_xor(c, o, kWave);
    m += __shfl_xor(m, o, kWave);
  }
  if (part == 0) {
    if (mode != kHistMass) h_cnt[b] = static_cast<uint32_t>(c);
    h_mass[b] = mode == kHistCount ? 0ull : m;
  }
  __syncthreads();
}

__device__ inline unsigned long long wave_sum_u64(unsigned long long v) {
  return wave_reduce(v, [](unsigned long long a, unsigned long long b) { return a + b; });
}

__device__ inline uint32_t wave_max_u(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}
__device__ inline uint32_t wave_min_u(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return min(a, b); });
}

__device__ inline void clear_columns(unsigned long long *lh) {
  for (int i = threadIdx.x; i < 256 * kWave; i += kProcThreads) lh[i] = 0ull;
}

// Lane t owns bucket nb - 1 - t (descending buckets in lane order; lanes past
// the buckets pass 0).  Returns the sum of v over the lanes before this one:
// for a bucket lane, the sum over the buckets above its own.  `sh` holds one
// word per wave.  Every lane of the block must call it (barriers).
__device__ inline unsigned long long sum_above(unsigned long long v, unsigned long long *sh) {
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const unsigned long long inc = wave_incl_scan(v);
  if (lane == kWave - 1) sh[w] = inc;
  __syncthreads();
  unsigned long long base = 0;
  for (int i = 0; i < w; ++i) base += sh[i];
  __syncthreads();
  return base + inc - v;
}

// Largest value of x over the block (x >= -1), broadcast.  Barriers.
__device__ inline int block_max_int(int x, int *sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  x = wave_max_i(x);
  if (lane == 0) sh[w] = x;
  __syncthreads();
  int r = sh[0];
  for (int i = 1; i < kProcWaves; ++i) r = max(r, sh[i]);
  __syncthreads();
  return r;
}

static_assert(kCandCap == 256 * kWave * 2, "the candidate list reuses the histogram's LDS");

// The float a (non-NaN) order key stands for; -0 comes back as +0, which is
// equal to it in every comparison and weight.
__device__ inline float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Appends the lanes with `want` set, in lane order, at a counter in LDS: one
// atomic per wave.  Every lane of the wave must call it; returns the lane's
// slot (meaningful where `want`).
__device__ inline int wave_append(bool want, int *counter) {
  const unsigned long long mask = __ballot(want);
  const int lane = threadIdx.x & (kWave - 1);
  int base = 0;
  if (mask != 0ull) {
    const int leader = __ffsll(static_cast<long long>(mask)) - 1;
    if (lane == leader) base = atomicAdd(counter, __popcll(mask));
    base = read_lane(base, leader);
  }
  return base + __popcll(mask & ((1ull << lane) - 1ull));
}


// Radix levels of 8 bits from bit `top` down to bit `low` (the last one may
// be narrower).  Keys in [klo, khi] share every bit above the highest bit in
// which klo and khi differ, so a selection among them starts there: top is
// that bit, or low - 1 (no level at all) when they agree on every bit from
// low up.
__device__ inline int digit_top(uint32_t klo, uint32_t khi, int low) {
  const uint32_t d = klo ^ khi;
  return max(d != 0u ? 31 - static_cast<int>(__clz(d)) : -1, low - 1);
}
__device__ inline uint32_t bits_above(int top) { return top >= 31 ? 0u : (0xFFFFFFFFu << (top + 1)); }

// Statistics of a short top-k candidate list by one wave, with the choices
// of the workgroup-wide code below: the same radix digits, tie rules and
// exact fixed-point sums, in one wave so that no step waits at a workgroup
// barrier.  each(f) calls f(key) with the order key of every candidate of
// this lane (0: none); the candidates hold every logit at or above the row's
// K-th largest and the row's largest, and their keys lie in [klo, khi].  The
// digits start below the bits all candidates share (one level instead of two
// for most bf16 lists); the keys chosen are the same as with fixed digits.
// Lane l owns buckets 255 - 4l .. 252 - 4l (descending) of hc / hm.
template <bool BF16, class Each>
__device__ inline void wave_list_stats(Each &&each, uint32_t klo, uint32_t khi, float zmax, Temper invT, int K,
                                       bool topp_on, float top_p, uint32_t *hc, unsigned long long *hm,
                                       ProcStats &st) {
  constexpr int kLow = BF16 ? 16 : 0;            // bf16 keys carry no information below bit 16
  const int lane = threadIdx.x & (kWave - 1);
  auto clear = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hc[4 * lane + j] = 0u;
      hm[4 * lane + j] = 0ull;
    }
    __builtin_amdgcn_wave_barrier();
  };
  auto excl_scan_u64 = [&](unsigned long long v) { return wave_incl_scan(v) - v; };
  // ---- top-k: the K-th largest key, one digit per level
  const int ktop = digit_top(klo, khi, kLow);
  uint32_t kmask = bits_above(ktop), kprefix = klo & kmask;
  if (K > 0) {
    uint32_t need = static_cast<uint32_t>(K);
    for (int hi = ktop; hi >= kLow; hi -= 8) {
      const int shift = max(hi - 7, kLow);
      const uint32_t dmask = (2u << (hi - shift)) - 1u;
      clear();
      each([&](uint32_t key) {
        if (key != 0u && (key & kmask) == kprefix) atomicAdd(&hc[(key >> shift) & dmask], 1u);
      });
      __builtin_amdgcn_wave_barrier();
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hc[255 - 4 * lane - j];
      unsigned long long run = excl_scan_u64(static_cast<unsigned long long>(c[0] + c[1] + c[2] + c[3]));
      int found = -1;
      uint32_t rest = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (found < 0 && run < need && need <= run + c[j]) {
          found = 255 - 4 * lane - j;
          rest = need - static_cast<uint32_t>(run);
        }
        run += c[j];
      }
      const unsigned long long m = __ballot(found >= 0);
      const int src = __ffsll(static_cast<long long>(m)) - 1;
      const int b = read_lane(found, src);
      need = read_lane(rest, src);
      kprefix |= static_cast<uint32_t>(b) << shift;
      kmask |= dmask << shift;
    }
  }
  const uint32_t tau = K > 0 ? kprefix : 0u;
  // ---- top-p over the survivors: the lowest non-empty bucket whose heavier
  //      buckets weigh less than top_p times the total, one digit per level
  uint32_t theta = tau;
  if (topp_on) {
    const uint32_t plo = max(tau, klo);          // the survivors' keys lie in [plo, khi]
    const int ptop = digit_top(plo, khi, kLow);
    uint32_t pmask = bits_above(ptop), pprefix = plo & pmask;
    unsigned long long above = 0ull;
    double thr = 0.0;
    bool dead = false, first = true;
    for (int hi = ptop; hi >= kLow; hi -= 8) {
      const int shift = max(hi - 7, kLow);
      const uint32_t dmask = (2u << (hi - shift)) - 1u;
      clear();
      each([&](uint32_t key) {
        if (key != 0u && key >= tau && (key & pmask) == pprefix) {
          const uint32_t d = (key >> shift) & dmask;
          atomicAdd(&hc[d], 1u);
          atomicAdd(&hm[d], fixed_weight(proc_weight(f32_from_order_key(key), zmax, invT)));
        }
      });
      __builtin_amdgcn_wave_barrier();
      uint32_t c[4];
      unsigned long long mw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hc[255 - 4 * lane - j];
        mw[j] = hm[255 - 4 * lane - j];
      }
      const unsigned long long lsum = mw[0] + mw[1] + mw[2] + mw[3];
      unsigned long long run = excl_scan_u64(lsum);
      if (first) thr = static_cast<double>(top_p) * static_cast<double>(wave_sum_u64(lsum));   // every survivor
      first = false;
      int best = -1;
      unsigned long long sbest = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c[j] > 0u && static_cast<double>(above + run) < thr) {
          best = 4 * lane + j;
          sbest = run;
        }
        run += mw[j];
      }
      const int pos = wave_max_i(best);             // the lowest eligible bucket
      if (pos < 0) {
        dead = true;
        break;
      }
      above += read_lane(sbest, pos >> 2);
      pprefix |= static_cast<uint32_t>(255 - pos) << shift;
      pmask |= dmask << shift;
    }
    if (!dead) theta = pprefix;
  }
  // ---- kept weight and smallest kept logit
  unsigned long long acc = 0ull;
  float zlo = INFINITY;
  each([&](uint32_t key) {
    if (key != 0u && key >= theta) {
      const float z = f32_from_order_key(key);
      acc += fixed_weight(proc_weight(z, zmax, invT));
      zlo = fminf(zlo, z);
    }
  });
  acc = wave_sum_u64(acc);
  zlo = -wave_max_dpp(-zlo);
  const double mass = static_cast<double>(acc) / kFixScale;
  st.zmax = zmax;
  st.theta = theta;
  st.mass = mass;
  st.inv_mass = mass > 0.0 ? static_cast<float>(1.0 / mass) : 0.0f;
  st.zmin_kept = zlo;
}

// Wave 0 of the statistics kernel, top-k lists of at most kGatherS slices of
// at most one wave (64 entries) each: one round of loads (every slice's
// count, cut and bound, and the first 64 entries of every list, issued
// together), then the entries at or above lo = max(largest cut, smallest
// bound) are appended to `cand` in lane order.  lo is at most the row's K-th
// largest key: some slice's cut is at most its own K-th largest, and the
// slices' bounds put ceil(K / S) * S >= K entries at or above the smallest.
// So `cand` holds every logit at or above the row's K-th largest, and the
// row's largest.  Returns the count (zmax: the largest), or -1 when the lists
// do not fit this shape (nothing written).
__device__ inline int wave_gather_topk(const ProcParams &P, int r, float *cand, float &zmax, uint32_t &klo,
                                       uint32_t &khi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int S = P.S;
  if (S > kGatherS || P.list_lb == nullptr) return -1;
  const size_t rs = static_cast<size_t>(r) * S;
  int cnt = 0;
  uint32_t cut = 0u, lb = 0xFFFFFFFFu;
  if (lane < S) {
    cnt = P.list_cnt[rs + lane];
    cut = P.list_cut[rs + lane];
    lb = P.list_lb[rs + lane];
  }
  // entry `lane` of every list (inside its segment: seg_cap >= 512 > lane)
  const uint32_t *base = reinterpret_cast<const uint32_t *>(P.lists) + static_cast<size_t>(r) * kCandCap + lane;
  uint32_t raw[kGatherS];
#pragma unroll
  for (int q = 0; q < kGatherS; ++q) raw[q] = q < S ? base[static_cast<size_t>(q) * P.seg_cap] : 0u;
  if (__ballot(cnt > kWave) != 0ull) return -1;
  const uint32_t lo = max(wave_max_u(cut), wave_min_u(lb));
  const unsigned long long below = (1ull << lane) - 1ull;
  int n = 0;            // uniform
  uint32_t mk = 0u;
#pragma unroll
  for (int q = 0; q < kGatherS; ++q) {
    if (q < S) {
      const uint32_t k = lane < read_lane(cnt, q) ? f32_order_key(__uint_as_float(raw[q])) : 0u;
      const bool keep = k != 0u && k >= lo;
      const unsigned long long m = __ballot(keep);
      if (keep) {
        cand[n + __popcll(m & below)] = f32_from_order_key(k);
        mk = max(mk, k);
      }
      n += __popcll(m);
    }
  }
  khi = wave_max_u(mk);
  klo = min(max(lo, 1u), khi);
  zmax = f32_from_order_key(khi);
  return n;
}

// Statistics of row r by one workgroup of kProcThreads lanes: stored at
// P.stats[r] and returned, both by lane 0 (other lanes return zeros).  lh:
// the workgroup's per-lane histogram columns (256 * kWave words of LDS),
// reused as the candidate list.
template <bool BF16>
__device__ __forceinline__ ProcStats proc_row_stats(const ProcParams &P, int r, unsigned long long *lh) {
  ProcStats res = {};
  __shared__ uint32_t h_cnt[kProcThreads];     // one bucket per lane (10-bit digits on lists)
  __shared__ unsigned long long h_mass[kProcThreads];
  __shared__ float sh_f[kProcWaves];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_need, sh_ncand, sh_n;
  __shared__ unsigned long long sh_above, sh_tot;
  __shared__ unsigned long long sh4[kProcWaves];
  __shared__ int sh_i[kProcWaves];
  __shared__ unsigned long long sh_u[kProcWaves];
  __shared__ int sh_seg[kSliceMaxS + 1];
  __shared__ uint32_t sh_cutw[kSliceMaxS];
  __shared__ uint32_t sh_lbw[kSliceMaxS];
  __shared__ unsigned long long sh_stot[kSliceMaxS];
  __shared__ uint32_t sh_smax[kSliceMaxS];
  __shared__ uint32_t sh_mk;
  __shared__ unsigned long long sh_rowtot;
  __shared__ bool sh_fast;
  __shared__ ProcStats sh_st;

  static_assert(kProcThreads == 4 * 256, "fold_columns assigns 4 lanes per bucket");
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int V = P.V;
  const void *row = proc_row<BF16>(P, r);
  const Temper invT = P.cfg.invT;
  const int K = P.cfg.top_k;
  const bool topk = K > 0 && K < V;
  const bool topp = P.cfg.top_p < 1.0f;
  const unsigned long long one = 1ull << kCntShift;
  float *cand = reinterpret_cast<float *>(lh);
  // counts and weights share one histogram word only while no lane column can
  // receive more than kPackedMaxColumn logits (16 threads per column, each at
  // most ceil(V / VEC / kProcThreads) vectors, plus one head and one tail entry)
  constexpr int kVecElems = BF16 ? 8 : 4;
  const bool packed = kProcWaves * ((V / kVecElems + kProcThreads - 1) / kProcThreads) * kVecElems + 2 <=
                      kPackedMaxColumn;

  // ---- the row's candidates: with top-k, the slice kernel's lists when every
  //      slice's fit (their union holds every logit at or above the K-th
  //      largest, and the largest); else pass 1 over the row: maximum, and the
  //      first top-k digit histogram
  // ---- temperature only, through the slice kernels: every logit is kept, so
  //      the slices' maxima, exact weights and minima are the whole answer
  //      (one wave, one round of loads)
  if (P.sl_max != nullptr && !topk && !topp) {
    if (t < kWave) {
      uint32_t mx = 0u, mn = 0xFFFFFFFFu;
      unsigned long long tot = 0ull;
      for (int q = lane; q < P.S; q += kWave) {
        const size_t i = static_cast<size_t>(r) * P.S + q;
        mx = max(mx, P.sl_max[i]);
        mn = min(mn, P.sl_min[i]);
        tot += P.sl_tot[i];
      }
      mx = wave_max_u(mx);
      mn = wave_min_u(mn);
      tot = wave_sum_u64(tot);
      if (t == 0) {
        ProcStats st;
        st.zmax = f32_from_order_key(mx);
        st.theta = 0u;
        st.mass = static_cast<double>(tot) / kFixScale;
        st.inv_mass = st.mass > 0.0 ? static_cast<float>(1.0 / st.mass) : 0.0f;
        st.zmin_kept = f32_from_order_key(mn);
        P.stats[r] = st;
        res = st;
        sh_st = st;
      }
    }
    if (P.probs) {
      __syncthreads();
      const ProcStats st = sh_st;
      float *out = P.probs + static_cast<size_t>(r) * V;
      row_foreach<BF16>(row, V, [&](int v, float z) { out[v] = proc_prob(z, st, invT); });
    }
    return res;
  }

  // ---- top-k lists of one wave per slice: wave 0 gathers the candidates
  //      and decides everything, with no workgroup barrier before the result
  if (P.lists && topk) {
    if (t < kWave) {
      float zm;
      uint32_t klo, khi;
      const int n = wave_gather_topk(P, r, cand, zm, klo, khi);
      if (n >= 0) {
        ProcStats st;
        wave_list_stats<BF16>(
            [&](auto &&f) {
              for (int i = lane; i < n; i += kWave) f(f32_order_key(cand[i]));
            },
            klo, khi, zm, invT, K, topp && zm != -INFINITY, P.cfg.top_p, h_cnt, h_mass, st);
        if (t == 0) sh_st = st;
      }
      if (t == 0) sh_fast = n >= 0;
    }
    __syncthreads();
    if (sh_fast) {
      const ProcStats st = sh_st;
      if (t == 0) {
        P.stats[r] = st;
        res = st;
      }
      if (P.probs) {
        float *out = P.probs + static_cast<size_t>(r) * V;
        row_foreach<BF16>(row, V, [&](int v, float z) { out[v] = proc_prob(z, st, invT); });
      }
      return res;
    }
  }

  bool fast = false;
  int nfast = 0;
  uint32_t cutmax = 0;
  // rows without top-k through the slice kernels: the maximum (and the exact
  // weight) from the slices
  const bool smode = P.sl_max != nullptr && !topk;
  float m = -INFINITY;
  bool have_slices = false;                      // sh_mk / sh_rowtot hold the slices' maximum and weight
  if (P.lists && (topk || (P.sl_max != nullptr && topp))) {
    // segment offsets (prefix of the list lengths) and the largest slice cut;
    // in slice mode the slices' maxima and weights come in the same round
    if (t < P.S) {
      const size_t i = static_cast<size_t>(r) * P.S + t;
      const int c = P.list_cnt[i];
      sh_seg[t] = c;
      sh_cutw[t] = P.list_cut[i];
      sh_lbw[t] = topk && P.list_lb ? P.list_lb[i] : 0u;
      if (smode) {
        sh_smax[t] = P.sl_max[i];
        sh_stot[t] = P.sl_tot[i];
      }
    }
    __syncthreads();
    if (t == 0) {
      int off = 0;
      uint32_t cm = 0, lbm = 0xFFFFFFFFu, mk = 0u;
      unsigned long long tw = 0ull;
      bool ok = true;
      for (int q = 0; q < P.S; ++q) {
        const int c = sh_seg[q];
        ok = ok && c <= P.seg_cap;
        sh_seg[q] = off;
        off += c;
        cm = max(cm, sh_cutw[q]);
        lbm = min(lbm, sh_lbw[q]);
        if (smode) {
          mk = max(mk, sh_smax[q]);
          tw += sh_stot[q];
        }
      }
      sh_seg[P.S] = off;
      sh_fast = ok;
      sh_cutw[0] = max(cm, lbm);     // with top-k: also the smallest slice bound
      sh_mk = mk;
      sh_rowtot = tw;
      sh_n = 0;
    }
    __syncthreads();
    fast = sh_fast;
    cutmax = sh_cutw[0];
    have_slices = smode;
  }
  if (smode) {
    uint32_t mk = 0;
    if (have_slices)
      mk = sh_mk;
    else
      for (int q = 0; q < P.S; ++q) mk = max(mk, P.sl_max[static_cast<size_t>(r) * P.S + q]);
    m = f32_from_order_key(mk);
  }
  if (fast) {
    // every slice's cut is at most the row's K-th largest key: entries below
    // the largest cut cannot be kept.  kCopyU independent loads per lane are
    // issued before any entry is appended.
    constexpr int kCopyU = 4;
    const int tot = sh_seg[P.S];
    for (int g0 = 0; g0 < tot; g0 += kProcThreads * kCopyU) {   // same trip count in every lane
      float z[kCopyU];
#pragma unroll
      for (int u = 0; u < kCopyU; ++u) {
        const int g = g0 + u * kProcThreads + t;
        z[u] = 0.0f;
        if (g < tot) {
          int q = 0;
          while (sh_seg[q + 1] <= g) ++q;
          z[u] = P.lists[static_cast<size_t>(r) * kCandCap + static_cast<size_t>(q) * P.seg_cap + (g - sh_seg[q])];
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyU; ++u) {
        const int g = g0 + u * kProcThreads + t;
        const bool keep = g < tot && f32_order_key(z[u]) >= cutmax;
        const int slot = wave_append(keep, &sh_n);
        if (keep) {
          cand[slot] = z[u];
          m = fmaxf(m, z[u]);
        }
      }
    }
  } else if (!smode) {
    clear_columns(lh);
    __syncthreads();
    row_foreach<BF16>(row, V, [&](int, float z) {
      m = fmaxf(m, z);
      if (topk) atomicAdd(&lh[(f32_order_key(z) >> 24) * kWave + lane], 1ull);
    });
  }
  const float zmax = block_max_f(m, sh_f);     // (contains barriers)
  if (fast) nfast = sh_n;
  const bool topp_on = topp && zmax != -INFINITY;

  // ---- a short top-k list: one wave decides everything (no workgroup
  //      barriers).  (Top-p lists without top-k are longer; the workgroup
  //      code below is faster for them.)
  if (fast && topk && nfast <= kWaveList) {
    if (t < kWave) {
      ProcStats st;
      const uint32_t khi = f32_order_key(zmax);
      wave_list_stats<BF16>(
          [&](auto &&f) {
            for (int i = lane; i < nfast; i += kWave) f(f32_order_key(cand[i]));
          },
          min(max(cutmax, 1u), khi), khi, zmax, invT, K, topp_on, P.cfg.top_p, h_cnt, h_mass, st);
      if (t == 0) sh_st = st;
    }
    __syncthreads();
    const ProcStats st = sh_st;
    if (t == 0) {
      P.stats[r] = st;
      res = st;
    }
    if (P.probs) {
      float *out = P.probs + static_cast<size_t>(r) * V;
      row_foreach<BF16>(row, V, [&](int v, float z) { out[v] = proc_prob(z, st, invT); });
    }
    return res;
  }

  // Selection state.  Level-0 digits are chosen from whole-row histograms;
  // everything at or above the chosen level-0 bucket is then copied into LDS
  // (when it fits) and the remaining levels run on that list.
  uint32_t kprefix = 0, kmask = 0;   // top-k descent
  int need = K;
  uint32_t pprefix = 0, pmask = 0;   // top-p descent
  unsigned long long above = 0;
  double thr = 0.0;
  bool p_started = false, p_dead = false;
  // Digits from a top bit down to kLow (the last may be narrower): 8 bits on
  // whole-row histograms (256 buckets x 64 lane columns), 10 bits on LDS
  // lists (one bucket per lane).  Whole-row histograms start at bit 31; a
  // list whose keys lie in [klo, khi] starts below the bits they all share.
  constexpr int kLow = BF16 ? 16 : 0;            // bf16 keys carry no information below bit 16
  constexpr int kRowDigit = 8, kListDigit = 10;
  static_assert((1 << kListDigit) == kProcThreads, "one list bucket per lane");
  int k_hi = 31, p_hi = 31;                      // top bit of the next top-k / top-p digit
  const uint32_t khi = f32_order_key(zmax);
  auto list_top = [&](uint32_t klo) { return max(digit_top(min(max(klo, 1u), khi), khi, kLow), kLow + 7); };
  auto digit_mask = [](int hi, int shift) { return (2u << (hi - shift)) - 1u; };

  // Picks the top-k bucket at `shift` from h_cnt; returns the count of keys
  // in the chosen bucket and above.  Barriers.
  auto select_k = [&](int shift, uint32_t dmask) -> int {
    const int nb = static_cast<int>(dmask) + 1;
    const int tb = nb - 1 - t;
    const unsigned long long c = t < nb ? h_cnt[tb] : 0ull;
    const unsigned long long S = sum_above(c, sh4);
    if (t < nb && S < static_cast<unsigned long long>(need) && static_cast<unsigned long long>(need) <= S + c) {
      sh_need = need - static_cast<int>(S);
      sh_prefix = kprefix | (static_cast<uint32_t>(tb) << shift);
      sh_ncand = static_cast<int>(S + c);
    }
    __syncthreads();
    need = sh_need;
    kprefix = sh_prefix;
    kmask |= dmask << shift;
    const int n = sh_ncand;
    __syncthreads();
    return n;
  };
  // Picks the top-p bucket at `shift` from h_cnt / h_mass (level 0 also fixes
  // the threshold top_p * total); returns the count in the bucket and above.
  unsigned long long hist_total = 0;          // level 0: the weight the histogram saw
  auto select_p = [&](int shift, uint32_t dmask, bool first, unsigned long long row_total) -> int {
    const int nb = static_cast<int>(dmask) + 1;
    const int tb = nb - 1 - t;
    const unsigned long long mw = t < nb ? h_mass[tb] : 0ull;
    const unsigned long long cw = t < nb ? h_cnt[tb] : 0ull;
    const unsigned long long S = sum_above(mw, sh4);
    const unsigned long long SC = sum_above(cw, sh4);
    if (first) {
      if (t == nb - 1) sh_tot = S + mw;
      __syncthreads();
      hist_total = sh_tot;
      thr = static_cast<double>(P.cfg.top_p) * static_cast<double>(row_total ? row_total : hist_total);
    }
    const bool ok = t < nb && cw > 0 && static_cast<double>(above + S) < thr;
    const int win = block_max_int(ok ? t : -1, sh_i);   // largest lane = lowest bucket
    if (win < 0) {
      if (t == 0) sh_prefix = 0xFFFFFFFFu;
    } else if (t == win) {
      sh_prefix = pprefix | (static_cast<uint32_t>(tb) << shift);
      sh_above = above + S;
      sh_ncand = static_cast<int>(SC + cw);
    }
    __syncthreads();
    const uint32_t np = sh_prefix;
    const int n = sh_ncand;
    if (np == 0xFFFFFFFFu) {
      p_dead = true;                              // no weight at all: keep the top-k set
    } else {
      pprefix = np;
      above = sh_above;
      pmask |= dmask << shift;
    }
    __syncthreads();
    return n;
  };

  int ncand = V;
  uint32_t cutoff = 0;
  bool use_list = fast && topk;                // every level runs on the slice lists
  if (fast && topk) {
    // every top-k level, the first included, runs on the list below, whose
    // keys lie in [cutmax, khi]
    k_hi = list_top(cutmax);
    kmask = bits_above(k_hi);
    kprefix = min(max(cutmax, 1u), khi) & kmask;
  } else if (topk) {
    fold_columns(lh, h_cnt, h_mass, kHistCount);
    ncand = select_k(24, 255u);
    k_hi = 23;
    cutoff = kprefix;
  } else if (topp_on) {
    if (fast) {
      // slice mode: the union of the lists holds every logit at or above the
      // largest slice cut.  Level 0 from the union's histogram, with the
      // threshold from the row's exact weight; valid when the union itself
      // weighs at least top_p of the row (then no logit outside it is kept).
      const unsigned long long row_total = sh_rowtot;   // read with the lists (slice mode)
      h_cnt[t] = 0u;                             // one bucket per lane
      h_mass[t] = 0ull;
      const int top = list_top(cutmax);          // the union's keys lie in [cutmax, khi]
      const int shift = max(top - (kListDigit - 1), kLow);
      const uint32_t dmask = digit_mask(top, shift);
      pmask = bits_above(top);
      pprefix = min(max(cutmax, 1u), khi) & pmask;
      __syncthreads();
      for (int i = t; i < nfast; i += kProcThreads) {
        const float z = cand[i];
        const uint32_t d = (f32_order_key(z) >> shift) & dmask;
        atomicAdd(&h_cnt[d], 1u);
        atomicAdd(&h_mass[d], fixed_weight(proc_weight(z, zmax, invT)));
      }
      __syncthreads();
      ncand = select_p(shift, dmask, true, row_total);
      if (!p_dead && static_cast<double>(hist_total) >= thr) {
        use_list = true;
        p_started = true;
        p_hi = shift - 1;
        cutoff = pprefix;
      } else {                                   // read the row after all
        p_dead = false;
        pprefix = pmask = 0u;
        above = 0ull;
      }
    }
    if (!use_list) {
      // pass 2 over the row: first top-p digit histogram (counts and weights;
      // counts, then weights, when a packed column could overflow)
      clear_columns(lh);
      __syncthreads();
      row_foreach<BF16>(row, V, [&](int, float z) {
        const uint32_t key = f32_order_key(z);
        atomicAdd(&lh[(key >> 24) * kWave + lane], packed ? one + fixed_weight(proc_weight(z, zmax, invT)) : 1ull);
      });
      __syncthreads();
      fold_columns(lh, h_cnt, h_mass, packed ? kHistPacked : kHistCount);
      if (!packed) {
        clear_columns(lh);
        __syncthreads();
        row_foreach<BF16>(row, V, [&](int, float z) {
          atomicAdd(&lh[(f32_order_key(z) >> 24) * kWave + lane], fixed_weight(proc_weight(z, zmax, invT)));
        });
        __syncthreads();
        fold_columns(lh, h_cnt, h_mass, kHistMass);
      }
      ncand = select_p(24, 255u, true, 0ull);
      p_started = true;
      p_hi = 23;
      if (!p_dead) cutoff = pprefix;
    }
  }
  const bool listed = use_list || ((topk || (topp_on && !p_dead)) && ncand <= kCandCap);
  int n = use_list ? nfast : 0;
  if (listed && !use_list) {
    // pass over the row: copy every logit at or above the cutoff into LDS
    // (ncand counted them; the bound keeps every write inside the list)
    if (t == 0) sh_n = 0;
    __syncthreads();
    row_foreach<BF16>(row, V, [&](int, float z) {
      if (f32_order_key(z) >= cutoff) {
        const int slot = atomicAdd(&sh_n, 1);
        if (slot < kCandCap) cand[slot] = z;
      }
    });
    __syncthreads();
    n = sh_n;
  }
  // A list that did not fit (the histogram's count was exact, so this does
  // not happen) is dropped: the remaining levels then read the row.
  const bool listed_ok = !(listed && !use_list) || n <= kCandCap;

  // Visits every logit that can still matter: the LDS list, or the row.
  const bool on_list = listed && listed_ok;
  auto each = [&](auto &&f) {
    if (on_list) {
      for (int i = t; i < n; i += kProcThreads) f(cand[i]);
    } else {
      row_foreach<BF16>(row, V, [&](int, float z) { f(z); });
    }
  };
  // Histogram of digit (key >> shift) & dmask over the logits passing `pred`,
  // with weights if asked, into h_cnt / h_mass.  Barriers.
  auto histogram = [&](int shift, uint32_t dmask, bool weights, auto &&pred) {
    if (on_list) {
      h_cnt[t] = 0u;                             // one bucket per lane
      h_mass[t] = 0ull;
      __syncthreads();
      each([&](float z) {
        const uint32_t key = f32_order_key(z);
        if (pred(key)) {
          const uint32_t d = (key >> shift) & dmask;
          atomicAdd(&h_cnt[d], 1u);
          if (weights) atomicAdd(&h_mass[d], fixed_weight(proc_weight(z, zmax, invT)));
        }
      });
      __syncthreads();
    } else {
      // whole-row words: counts alone, counts and weights packed, or (when a
      // packed column could overflow) a pass of counts and a pass of weights
      const HistMode first = !weights ? kHistCount : (packed ? kHistPacked : kHistCount);
      clear_columns(lh);
      __syncthreads();
      each([&](float z) {
        const uint32_t key = f32_order_key(z);
        if (pred(key)) {
          const unsigned long long add =
              first == kHistPacked ? one + fixed_weight(proc_weight(z, zmax, invT)) : 1ull;
          atomicAdd(&lh[((key >> shift) & dmask) * kWave + lane], add);
        }
      });
      __syncthreads();
      fold_columns(lh, h_cnt, h_mass, first);
      if (weights && !packed) {
        clear_columns(lh);
        __syncthreads();
        each([&](float z) {
          const uint32_t key = f32_order_key(z);
          if (pred(key)) atomicAdd(&lh[((key >> shift) & dmask) * kWave + lane], fixed_weight(proc_weight(z, zmax, invT)));
        });
        __syncthreads();
        fold_columns(lh, h_cnt, h_mass, kHistMass);
      }
    }
  };

  // ---- top-k: remaining digits
  uint32_t tau = 0;
  const int digit = on_list ? kListDigit : kRowDigit;
  if (topk) {
    for (int hi = k_hi; hi >= kLow; hi -= digit) {
      const int shift = max(hi - (digit - 1), kLow);
      const uint32_t dmask = digit_mask(hi, shift);
      const uint32_t pf = kprefix, pm = kmask;
      histogram(shift, dmask, false, [&](uint32_t key) { return (key & pm) == pf; });
      select_k(shift, dmask);
    }
    tau = kprefix;   // the smallest key with the selected significant bits
  }

  // ---- top-p over the top-k survivors
  uint32_t theta = tau;
  if (topp_on) {
    if (!p_started && topk) {                    // the survivors' keys lie in [tau, khi]
      p_hi = list_top(tau);
      pmask = bits_above(p_hi);
      pprefix = min(max(tau, 1u), khi) & pmask;
    }
    bool first = !p_started;
    for (int hi = p_hi; hi >= kLow && !p_dead; hi -= digit) {
      const int shift = max(hi - (digit - 1), kLow);
      const uint32_t dmask = digit_mask(hi, shift);
      const uint32_t pf = pprefix, pm = pmask, tk = tau;
      histogram(shift, dmask, true, [&](uint32_t key) { return key >= tk && (key & pm) == pf; });
      select_p(shift, dmask, first, 0ull);
      first = false;
    }
    if (!p_dead) theta = pprefix;
  }

  // ---- kept weight (exact integer sum of fixed-point weights, so any visiting
  //      order gives the same bits) and the smallest kept logit
  unsigned long long acc = 0;
  float zlo = INFINITY;
  if (smode && theta == 0u) {
    // every entry is kept: the slices' weights and smallest keys
    if (t == 0) {
      for (int q = 0; q < P.S; ++q) {
        acc += P.sl_tot[static_cast<size_t>(r) * P.S + q];
        zlo = fminf(zlo, f32_from_order_key(P.sl_min[static_cast<size_t>(r) * P.S + q]));
      }
    }
  } else {
    each([&](float z) {
      if (f32_order_key(z) >= theta) {
        acc += fixed_weight(proc_weight(z, zmax, invT));
        zlo = fminf(zlo, z);
      }
    });
  }
  {
    acc = wave_sum_u64(acc);
    if (lane == 0) sh_u[t / kWave] = acc;
    __syncthreads();
    unsigned long long tot = 0;
    for (int i = 0; i < kProcWaves; ++i) tot += sh_u[i];
    acc = tot;
    __syncthreads();
  }
  const double mass = static_cast<double>(acc) / kFixScale;
  const float zmin_kept = -block_max_f(-zlo, sh_f);
  ProcStats st;
  st.zmax = zmax;
  st.theta = theta;
  st.mass = mass;
  st.inv_mass = mass > 0.0 ? static_cast<float>(1.0 / mass) : 0.0f;
  st.zmin_kept = zmin_kept;
  if (t == 0) {
    P.stats[r] = st;
    res = st;
  }
  if (P.probs) {
    float *out = P.probs + static_cast<size_t>(r) * V;
    row_foreach<BF16>(row, V, [&](int v, float z) { out[v] = proc_prob(z, st, invT); });
  }
  return res;
}

template <bool BF16>
__global__ __launch_bounds__(kProcThreads) void proc_stats_kernel(ProcParams P) {
  __shared__ unsigned long long lh[256 * kWave];
  (void)proc_row_stats<BF16>(P, blockIdx.x, lh);
}

// Slice s of row r: kSliceThreads * kSliceLoads 16-byte vectors; lane t
// owns vectors u * kSliceThreads + t (u < kSliceLoads), whose entry e is entry
// (u * kSliceThreads + t) * VEC + e of the slice.  The kernels below work on
// the raw vectors: the float value of an entry is one shift or mask away,
// and float maxima and minima agree with the order keys (f32_order_key is
// monotone and maps -0 and +0 to one key).
template <bool BF16>
struct Slice {
  static constexpr int VEC = BF16 ? 8 : 4;                 // entries per vector
  static constexpr int SL = kSliceThreads * kSliceLoads * VEC;
  const unsigned char *base;   // first entry of the slice
  int n;                       // entries in the slice
  bool vec;                    // 16-byte aligned: whole vectors load as they are

  __device__ Slice(const ProcParams &P, int r, int s) {
    const int v0 = s * SL;
    n = min(P.V - v0, SL);
    base = static_cast<const unsigned char *>(proc_row<BF16>(P, r)) + static_cast<size_t>(v0) * (BF16 ? 2 : 4);
    vec = (reinterpret_cast<uintptr_t>(base) & 15u) == 0;
  }
  __device__ int first(int u) const { return (u * kSliceThreads + static_cast<int>(threadIdx.x)) * VEC; }
  __device__ bool whole(int u) const { return vec && first(u) + VEC <= n; }
  // Every vector of this lane; an entry past the row reads as -inf.
  __device__ void load(uint4 (&q)[kSliceLoads]) const {
#pragma unroll
    for (int u = 0; u < kSliceLoads; ++u) {
      const int i0 = first(u);
      if (whole(u)) {
        q[u] = reinterpret_cast<const uint4 *>(base)[u * kSliceThreads + threadIdx.x];
      } else {
        uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t x = __float_as_uint(i0 + e < n ? logit_at<BF16>(base, i0 + e) : -INFINITY);
          if constexpr (BF16)
            wd[e >> 1] |= (e & 1) ? (x & 0xFFFF0000u) : (x >> 16);
          else
            wd[e] = x;
        }
        q[u] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
  }
};

// Entry e of a loaded vector as a float.
template <bool BF16>
__device__ inline float vec_entry(const uint4 &q, int e) {
  const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
  if constexpr (BF16)
    return __uint_as_float((e & 1) ? (wd[e >> 1] & 0xFFFF0000u) : (wd[e >> 1] << 16));
  else
    return __uint_as_float(wd[e]);
}

template <bool BF16>
__device__ inline float vec_max(const uint4 &q) {
  float m = vec_entry<BF16>(q, 0);
#pragma unroll
  for (int e = 1; e < Slice<BF16>::VEC; ++e) m = fmaxf(m, vec_entry<BF16>(q, e));
  return m;
}

// Top-k candidates of one slice.  Each lane takes the float maximum of each
// of its vectors and of all of them; theta is the K-th largest of the 256
// lane maxima (as order keys).  At least K entries (those maxima) are at or
// above theta, so theta is at most the slice's K-th largest key, and the
// slice lists every entry at or above it.  A logit at or above the row's K-th
// largest is among the K largest of its slice, so the union of the slices'
// lists holds all of them, and no slice's theta exceeds the row's K-th
// largest key.  Listing: the vectors whose maximum reaches theta (about K of
// them) are staged in LDS and the whole workgroup filters their entries, so
// only those vectors are looked at twice; when more than kStageCap qualify
// every lane filters its own.  A list that does not fit reports its length;
// the statistics kernel then reads the row whole.  (K <= 256.)
constexpr int kStageCap = 512;
static_assert(kSliceThreads == 4 * kWave, "four lane maxima per lane of a wave");

// The r1-th and r2-th largest (1 <= r <= 256, counting repeats) of the 256
// keys m, four per lane, every lane of the wave active, and the largest key:
// for each rank, the largest c with at least r keys >= c, decided one bit at
// a time by counting the keys >= the candidate with wave ballots.  Every key
// shares the bits above the highest bit in which the smallest and the largest
// differ, so the search starts below them.  Keys of bf16 logits (kLow = 16)
// carry nothing below bit 16: keys with equal top halves are equal, their low
// half all zeros for a non-negative logit (and for the key 0 of a lane with no
// entry) and all ones for a negative one, so only the top 16 bits are searched
// and the low half is filled in.  With two == false only r1 is searched.
template <int kLow>
__device__ inline void kth_keys(const uint32_t (&m)[4], int r1, int r2, bool two, uint32_t &x1, uint32_t &x2,
                                uint32_t &kmax) {
  const uint32_t hi = wave_max_u(max(max(m[0], m[1]), max(m[2], m[3])));
  const uint32_t lo = wave_min_u(min(min(m[0], m[1]), min(m[2], m[3])));
  const int top = digit_top(lo, hi, kLow);
  uint32_t p1 = lo & bits_above(top), p2 = p1;
  if (two) {
    for (int b = top; b >= kLow; --b) {
      const uint32_t c1 = p1 | (1u << b), c2 = p2 | (1u << b);
      int n1 = 0, n2 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        n1 += __popcll(__ballot(m[i] >= c1));
        n2 += __popcll(__ballot(m[i] >= c2));
      }
      if (n1 >= r1) p1 = c1;
      if (n2 >= r2) p2 = c2;
    }
  } else {
    for (int b = top; b >= kLow; --b) {
      const uint32_t c1 = p1 | (1u << b);
      int n1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) n1 += __popcll(__ballot(m[i] >= c1));
      if (n1 >= r1) p1 = c1;
    }
    p2 = p1;
  }
  if constexpr (kLow == 16) {
    if (p1 != 0u && p1 < 0x80000000u) p1 |= 0xFFFFu;
    if (p2 != 0u && p2 < 0x80000000u) p2 |= 0xFFFFu;
  }
  x1 = p1;
  x2 = p2;
  kmax = hi;
}

template <bool BF16>
__global__ __launch_bounds__(kSliceThreads) void proc_slice_kernel(ProcParams P) {
  using SV = Slice<BF16>;
  constexpr int VEC = SV::VEC;
  __shared__ uint32_t sh_m[kSliceThreads];
  __shared__ uint4 sh_vec[kStageCap];
  __shared__ uint16_t sh_vid[kStageCap];
  __shared__ int sh_nv, sh_n;
  const int t = threadIdx.x, lane = t & (kWave - 1);
  const int r = blockIdx.x / P.S, s = blockIdx.x - r * P.S;
  const int K = P.cut_rank;
  const SV sl(P, r, s);
  uint4 q[kSliceLoads];
  sl.load(q);
  float fm[kSliceLoads];
  float fl = -INFINITY;
#pragma unroll
  for (int u = 0; u < kSliceLoads; ++u) {
    fm[u] = vec_max<BF16>(q[u]);
    fl = fmaxf(fl, fm[u]);
  }
  const uint32_t ml = sl.first(0) < sl.n ? f32_order_key(fl) : 0u;   // 0: a lane with no entry
  if (t == 0) {
    sh_nv = 0;
    sh_n = 0;
  }
  // every wave reads all 256 lane maxima and finds the ranks it needs itself
  sh_m[t] = ml;
  __syncthreads();
  uint32_t m4[kSliceThreads / kWave];
#pragma unroll
  for (int i = 0; i < kSliceThreads / kWave; ++i) m4[i] = sh_m[lane + i * kWave];
  uint32_t theta, lb, smax;
  kth_keys<BF16 ? 16 : 0>(m4, K, P.lb_rank, P.list_lb != nullptr, theta, lb, smax);
  if (t == 0) {
    if (P.sl_max) P.sl_max[static_cast<size_t>(r) * P.S + s] = smax;   // the slice's largest key
    if (P.list_lb) P.list_lb[static_cast<size_t>(r) * P.S + s] = lb;
    if (P.row_pub && s == 0)                        // written by the next launch's statistics
      for (int i = 0; i < 3; ++i) P.row_pub[3 * static_cast<size_t>(r) + i] = 0ull;
  }
  const uint32_t cut = max(theta, 1u);    // a maximum of 0 (no entry) lists every entry
  // a vector holds a key >= cut iff its float maximum is >= the cut's value
  // (every real key is at least the key of -inf)
  const float cutf = cut <= f32_order_key(-INFINITY) ? -INFINITY : f32_from_order_key(cut);
  const int cap = P.seg_cap;
  const size_t seg = static_cast<size_t>(r) * kCandCap + static_cast<size_t>(s) * cap;
  float *out = P.lists + seg;
  int32_t *out_idx = P.list_idx ? P.list_idx + seg : nullptr;
  const int v0 = s * SV::SL;                    // the slice's first index in the row
  bool stage[kSliceLoads];
  int c = 0;
#pragma unroll
  for (int u = 0; u < kSliceLoads; ++u) {
    stage[u] = fm[u] >= cutf && sl.first(u) < sl.n;
    c += stage[u];
  }
  // stage this lane's qualifying vectors at a wave-wide prefix sum
  const int x = wave_incl_scan(c);
  const int wtot = read_lane(x, kWave - 1);
  int pos = 0;
  if (wtot != 0) {
    if (lane == kWave - 1) pos = atomicAdd(&sh_nv, wtot);
    pos = read_lane(pos, kWave - 1);
  }
  pos += x - c;
#pragma unroll
  for (int u = 0; u < kSliceLoads; ++u) {
    if (stage[u]) {
      if (pos < kStageCap) {
        sh_vec[pos] = q[u];
        sh_vid[pos] = static_cast<uint16_t>(u * kSliceThreads + t);
      }
      ++pos;
    }
  }
  __syncthreads();
  const int nv = sh_nv;
  if (nv <= kStageCap) {
    const int items = nv * VEC;
    for (int i0 = 0; i0 < items; i0 += kSliceThreads) {     // same trip count in every lane
      const int i = i0 + t;
      uint32_t key = 0u;
      int ve = 0;                               // the entry's index in the slice
      if (i < items) {
        const int j = i / VEC, e = i - j * VEC;
        const uint32_t w = reinterpret_cast<const uint32_t *>(&sh_vec[j])[BF16 ? (e >> 1) : e];
        const float z = __uint_as_float(BF16 ? ((e & 1) ? (w & 0xFFFF0000u) : (w << 16)) : w);
        ve = static_cast<int>(sh_vid[j]) * VEC + e;
        if (ve < sl.n) key = f32_order_key(z);
      }
      const bool want = key >= cut;
      const int p = wave_append(want, &sh_n);
      if (want && p < cap) {
        out[p] = f32_from_order_key(key);
        if (out_idx) out_idx[p] = v0 + ve;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kSliceLoads; ++u) {
      if (stage[u]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t key = sl.first(u) + e < sl.n ? f32_order_key(vec_entry<BF16>(q[u], e)) : 0u;
          if (key >= cut) {
            const int p = atomicAdd(&sh_n, 1);
            if (p < cap) {
              out[p] = f32_from_order_key(key);
              if (out_idx) out_idx[p] = v0 + sl.first(u) + e;
            }
          }
        }
      }
    }
  }
  __syncthreads();
  if (t == 0) {
    P.list_cnt[static_cast<size_t>(r) * P.S + s] = sh_n;
    P.list_cut[static_cast<size_t>(r) * P.S + s] = theta;
  }
}

// Rows without top-k or top-p, step 1: the largest key of each slice.
template <bool BF16>
__global__ __launch_bounds__(kSliceThreads) void proc_slrange_kernel(ProcParams P) {
  constexpr int NW = kSliceThreads / kWave;
  __shared__ uint32_t sh_hi[NW];
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int r = blockIdx.x / P.S, s = blockIdx.x - r * P.S;
  const Slice<BF16> sl(P, r, s);
  uint4 q[kSliceLoads];
  sl.load(q);
  float fl = -INFINITY;
#pragma unroll
  for (int u = 0; u < kSliceLoads; ++u) fl = fmaxf(fl, vec_max<BF16>(q[u]));
  uint32_t hi = wave_max_u(sl.first(0) < sl.n ? f32_order_key(fl) : 0u);
  if (lane == 0) sh_hi[w] = hi;
  __syncthreads();
  if (t == 0) {
    for (int i = 0; i < NW; ++i) hi = max(hi, sh_hi[i]);
    P.sl_max[static_cast<size_t>(r) * P.S + s] = hi;
  }
}

// Rows without top-k, step 2: the row maximum from the slices' maxima, then
// each slice's fixed-point weight (an exact integer sum) and smallest key.
// With a finite row maximum the weight of a -inf logit is exp2(-inf) = 0, as
// proc_weight gives it, so whole vectors need no test per entry; a lane sums
// the two 20-bit parts of its fixed-point weights in 32-bit words (at most 64
// entries of at most 2^20 each) and combines them once.
template <bool BF16>
__global__ __launch_bounds__(kSliceThreads) void proc_slmass_kernel(ProcParams P) {
  using SV = Slice<BF16>;
  constexpr int NW = kSliceThreads / kWave, VEC = SV::VEC;
  static_assert(kSliceLoads * VEC <= 64, "per-lane part sums fit 32 bits");
  __shared__ unsigned long long sh_t[NW];
  __shared__ uint32_t sh_lo[NW];
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int r = blockIdx.x / P.S, s = blockIdx.x - r * P.S;
  uint32_t mk = 0u;
  for (int j = 0; j < P.S; ++j) mk = max(mk, P.sl_max[static_cast<size_t>(r) * P.S + j]);
  const float zmax = f32_from_order_key(mk);
  const bool finite = zmax != -INFINITY;      // else every weight is 0
  const Temper invT = P.cfg.invT;
  const SV sl(P, r, s);
  uint4 q[kSliceLoads];
  sl.load(q);
  uint32_t sum_hi = 0u, sum_lo = 0u;
  float zlo = INFINITY;
#pragma unroll
  for (int u = 0; u < kSliceLoads; ++u) {
    if (sl.whole(u)) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) zlo = fminf(zlo, vec_entry<BF16>(q[u], e));
    } else {
      const int i0 = sl.first(u);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (i0 + e < sl.n) {
          const float z = vec_entry<BF16>(q[u], e);
          zlo = fminf(zlo, z);
          const unsigned long long f = finite ? fixed_weight(proc_weight(z, zmax, invT)) : 0ull;
          sum_hi += static_cast<uint32_t>(f >> 20);
          sum_lo += static_cast<uint32_t>(f & 0xFFFFFu);
        }
      }
    }
  }
  if (finite) {
#pragma unroll
    for (int u = 0; u < kSliceLoads; ++u) {
      if (sl.whole(u)) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float a = proc_weight(vec_entry<BF16>(q[u], e), zmax, invT) * 1048576.0f;
          const uint32_t hi = static_cast<uint32_t>(a);
          sum_hi += hi;
          sum_lo += static_cast<uint32_t>((a - static_cast<float>(hi)) * 1048576.0f);
        }
      }
    }
  }
  unsigned long long tot = wave_sum_u64((static_cast<unsigned long long>(sum_hi) << 20) + sum_lo);
  uint32_t lo = wave_min_u(sl.first(0) < sl.n ? f32_order_key(zlo) : 0xFFFFFFFFu);
  if (lane == 0) {
    sh_t[w] = tot;
    sh_lo[w] = lo;
  }
  __syncthreads();
  if (t == 0) {
    unsigned long long a = 0ull;
    for (int i = 0; i < NW; ++i) {
      a += sh_t[i];
      lo = min(lo, sh_lo[i]);
    }
    P.sl_tot[static_cast<size_t>(r) * P.S + s] = a;
    P.sl_min[static_cast<size_t>(r) * P.S + s] = lo;
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

// ---------------------------------------------------------------------------
// Statistics and stochastic verification in one launch (rows processed
// through the slice lists: top-k, or top-p alone).
//
// With top-k through the slice lists, every entry a processed row keeps (its
// order key at or above the row's threshold, itself at or above the row's
// K-th largest key) is in that row's lists whenever every list fit its
// segment.  Without top-k (top-p alone) the lists hold every entry at or
// above their slice's cut, so they hold the kept entries whenever the row's
// threshold reaches the largest cut (the finisher checks).  So the token
// drawn at the end of a round, from p'_j - q'_j (first rejection) or p'_k
// (all accepted), needs only the target row's kept entries (p'_j is zero
// elsewhere, so is the residual): the finisher takes them from the lists,
// orders them by index, and draws by the inverse CDF over them.
// After the slice launches (the slice kernel also clears each row's
// published words; top-p alone adds the slices' exact weights), one launch:
// the statistics workgroups, one per row, each publishing its row's
// statistics, and behind them (dispatch is in index order) one finisher per
// sequence and, with offsets, one offsets workgroup.  While the
// statistics are computed, a finisher loads everything that does not depend
// on them: the drafts, uniforms and budget, the logits at the drafted tokens,
// and the lengths and first 64 entries of every list of its k + 1 target
// rows.  Once its 2k + 1 rows are published it takes the tries (the rule and
// arithmetic of the other stochastic kernels), keeps the listed entries of
// the row drawn from that reach its threshold, orders them by index, gathers
// the draft's logits there (residual only) and draws.  A row whose lists
// overflowed, that the lists do not cover, or that keeps more than one entry
// per lane, is drawn from the whole rows instead (chunk masses, then one
// chunk scanned in index order).

struct ProcVerifyParams {
  ProcParams proc;   // statistics of rows [0, B(k+1)) target, [B(k+1), B(2k+1)) draft;
                     // proc.row_pub: cleared by the slice kernel, published here
  SampleParams smp;  // the verification (smp.sp / smp.sq unused: the statistics travel
                     // in proc.row_pub)
};

// A row's statistics travel as three 64-bit words written with agent-scope
// atomic stores, each carrying a pattern no value here takes, so that every
// published word is nonzero and a zero word means "not yet written": a NaN
// in the half that holds zmax (inv_mass), which are never NaN, and the NaN
// sentinel XOR-ed onto the mass (a finite non-negative double).
constexpr uint32_t kHalfSentinel = 0x7FC00001u;
constexpr unsigned long long kStatSentinel = 0x7FF4000000000001ull;
__device__ inline void publish_stats(unsigned long long *w, const ProcStats &st) {
  const unsigned long long w0 =
      (static_cast<unsigned long long>(__float_as_uint(st.zmax) ^ kHalfSentinel) << 32) | st.theta;
  const unsigned long long w1 = static_cast<unsigned long long>(__double_as_longlong(st.mass)) ^ kStatSentinel;
  const unsigned long long w2 =
      (static_cast<unsigned long long>(__float_as_uint(st.inv_mass) ^ kHalfSentinel) << 32) |
      __float_as_uint(st.zmin_kept);
  __hip_atomic_store(w + 0, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(w + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(w + 2, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Word f (0, 1, 2) of a row's statistics into st.
__device__ inline void unpack_stats(ProcStats &st, int f, unsigned long long w) {
  if (f == 0) {
    st.zmax = __uint_as_float(static_cast<uint32_t>(w >> 32) ^ kHalfSentinel);
    st.theta = static_cast<uint32_t>(w);
  } else if (f == 1) {
    st.mass = __longlong_as_double(static_cast<long long>(w ^ kStatSentinel));
  } else {
    st.inv_mass = __uint_as_float(static_cast<uint32_t>(w >> 32) ^ kHalfSentinel);
    st.zmin_kept = __uint_as_float(static_cast<uint32_t>(w));
  }
}

constexpr int kDenseChunk = kProcThreads * 16;                       // whole-row draw: entries per chunk
constexpr int kDenseMaxChunks = (SPEC_PROC_MAX_V + kDenseChunk - 1) / kDenseChunk;
constexpr int kPfPairs = 128;          // (target row, slice) lists whose head a finisher loads early
constexpr int kPfHead = kWave;         // entries of a list's head
constexpr int kMaxRows = 2 * SPEC_MAX_K + 1;
constexpr int kRankAll = 128;          // kept entries up to this many are ranked among all of them

// A finisher's LDS, carved from the statistics workgroups' histogram buffer
// (the two roles never share a workgroup).
struct FinishLds {
  float pf_val[kPfPairs * kPfHead];    // list heads: logits, indices
  int pf_idx[kPfPairs * kPfHead];
  ProcStats stat[kMaxRows];            // the sequence's rows: target 0..k, then draft 0..k-1
  int cnt[kPfPairs];                   // list lengths of the target rows (prefetched)
  int cnt_row[kSliceMaxS];             // list lengths of the row drawn from (when not prefetched)
  int idx[kProcThreads];               // kept entries: indices, logits and slices, in list order
  float val[kProcThreads];
  int qs[kProcThreads];
  int gidx[kProcThreads];              // ... grouped by slice
  float gval[kProcThreads];
  int gq[kProcThreads];
  int ord[kProcThreads];               // ... in index order
  float ordv[kProcThreads];
  int qn[kSliceMaxS];                  // kept entries per slice, their offsets, placement counters
  int qbase[kSliceMaxS];
  int qpos[kSliceMaxS];
  double cm[kDenseMaxChunks];          // whole-row draw: chunk masses
};
static_assert(sizeof(FinishLds) <= sizeof(unsigned long long) * 256 * kWave, "finisher LDS fits the histogram buffer");

// Workgroup reductions over kProcThreads lanes in a fixed order (lanes of a
// wave, then waves).  `sh` holds kProcWaves values; each contains barriers.
__device__ inline double pv_sum(double v, double *sh) {
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
// Inclusive prefix sum of v in lane order; *total: the workgroup's sum.
__device__ inline double pv_incl_scan(double v, double *sh, double *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const double inc = wave_incl_scan(v);
  if (lane == kWave - 1) sh[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < kProcWaves; ++i) {
    if (i < w) base += sh[i];
    tot += sh[i];
  }
  __syncthreads();
  *total = tot;
  return base + inc;
}
// The smallest a and the largest b over the workgroup (one exchange).
__device__ inline int2 pv_min_max(int a, int b, int2 *sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  a = wave_min(a);
  b = wave_max_i(b);
  if (lane == 0) sh[w] = make_int2(a, b);
  __syncthreads();
  int2 m = sh[0];
#pragma unroll
  for (int i = 1; i < kProcWaves; ++i) {
    m.x = min(m.x, sh[i].x);
    m.y = max(m.y, sh[i].y);
  }
  __syncthreads();
  return m;
}

// Draw from the whole row r (LogitRow: p'_j - q'_j or p'_j): chunk masses
// (16 consecutive entries per lane, in order), their sum S, the chunk whose
// running sum first exceeds u * S (else the last with mass), then that chunk
// scanned in index order.  Sets S (the mass drawn from) and st's bits as the
// other stochastic kernels do.
template <bool BF16>
__device__ __forceinline__ int pv_draw_dense(LogitRow<BF16> r, int V, bool vec, float u_draw, double &S, int &st,
                                             double *sh_cm, double *sh_d, int2 *sh_i) {
  const int t = threadIdx.x;
  const int nch = (V + kDenseChunk - 1) / kDenseChunk;
  auto masses = [&]() {
    for (int c = 0; c < nch; ++c) {
      float x[16];
      r.load16(x, c * kDenseChunk + t * 16, V, vec);
      double a = 0.0;
#pragma unroll
      for (int i = 0; i < 16; ++i) a += static_cast<double>(x[i]);
      a = pv_sum(a, sh_d);
      if (t == 0) sh_cm[c] = a;
    }
    __syncthreads();
    double tot = 0.0;
    for (int c = 0; c < nch; ++c) tot += sh_cm[c];
    return tot;
  };
  S = masses();
  if (isfinite(S) && !(S > 0.0)) {
    st |= SPEC_ST_RESID_ZERO;
    if (r.resid) {                      // fall back to the target row p'_j itself
      r.resid = false;
      __syncthreads();
      S = masses();
    }
  }
  if (!isfinite(S)) {
    st |= SPEC_ST_NONFINITE;
    return 0;
  }
  if (!(S > 0.0)) return 0;
  const double T = static_cast<double>(u_draw) * S;
  int cs = -1, last = -1;
  double base = 0.0, lbase = 0.0, run = 0.0;
  for (int c = 0; c < nch; ++c) {       // the same in every lane
    const double m = sh_cm[c];
    if (m > 0.0) {
      last = c;
      lbase = run;
    }
    if (run + m > T) {
      cs = c;
      base = run;
      break;
    }
    run += m;
  }
  if (cs < 0) {
    cs = last;
    base = lbase;
  }
  const int lo = cs * kDenseChunk + t * 16;
  float x[16];
  r.load16(x, lo, V, vec);
  double mine = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) mine += static_cast<double>(x[i]);
  double ctot;
  double acc = base + (pv_incl_scan(mine, sh_d, &ctot) - mine);
  int cpos = INT_MAX, lastpos = -1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int v = lo + i;
    if (v < V) {
      if (x[i] > 0.0f) lastpos = v;
      acc += static_cast<double>(x[i]);
      if (cpos == INT_MAX && acc > T) cpos = v;
    }
  }
  const int2 mm = pv_min_max(cpos, lastpos, sh_i);
  return mm.x != INT_MAX ? mm.x : mm.y;
}

// Finisher of sequence b (see above); lh: the workgroup's LDS buffer.
template <bool BF16>
__device__ __forceinline__ void pv_finish(const ProcVerifyParams &X, int b, unsigned long long *lh) {
  using Src = LogitSrc<BF16>;
  __shared__ int sh_acc[SPEC_MAX_K], sh_st[SPEC_MAX_K], sh_d[SPEC_MAX_K];
  __shared__ int4 sh_ch;
  __shared__ int sh_n;
  __shared__ unsigned sh_cutmax;
  __shared__ double sh_dw[kProcWaves];
  __shared__ int2 sh_iw[kProcWaves];
  FinishLds &L = *reinterpret_cast<FinishLds *>(lh);
  const SampleParams &P = X.smp;
  const ProcParams &Q = X.proc;
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int k = P.k, kp1 = k + 1, nr = 2 * k + 1, V = P.V;
  const int nS = Q.S, cap = Q.seg_cap;
  auto row_of = [&](int i) { return i < kp1 ? b * kp1 + i : P.B * kp1 + b * k + (i - kp1); };
  auto seg_of = [&](int j, int q) {            // list segment q of target row j
    return static_cast<size_t>(b * kp1 + j) * kCandCap + static_cast<size_t>(q) * cap;
  };

  // ---- before the statistics: drafts, uniforms, budget, logits at the
  //      drafted tokens, and the target rows' list lengths and heads
  const float u_draw = P.u[static_cast<size_t>(b) * kp1 + k];
  const int rem = P.remaining ? P.remaining[b] : -1;       // negative: no budget
  int x_t = -1;
  float u_t = 0.0f, zp_t = 0.0f, zq_t = 0.0f;
  if (t < k) {
    x_t = P.draft[static_cast<size_t>(b) * k + t];
    u_t = P.u[static_cast<size_t>(b) * kp1 + t];
    if (x_t >= 0 && x_t < V) {
      zp_t = logit_at<BF16>(Src::prow(P, b, t), x_t);
      zq_t = logit_at<BF16>(Src::qrow(P, b, t), x_t);
    }
  }
  const int npair = kp1 * nS;
  const bool pre = npair <= kPfPairs;
  if (pre) {
    if (t < npair) L.cnt[t] = Q.list_cnt[static_cast<size_t>(b * kp1 + t / nS) * nS + t % nS];
    for (int pr = w; pr < npair; pr += kProcWaves) {   // the head of every list (inside its segment)
      const size_t e = seg_of(pr / nS, pr % nS) + lane;
      L.pf_val[pr * kPfHead + lane] = Q.lists[e];
      L.pf_idx[pr * kPfHead + lane] = Q.list_idx[e];
    }
  }

  // ---- the statistics of the sequence's 2k + 1 rows (bounded wait); they
  //      arrive in the published words themselves
  const int nwords = 3 * nr;
  unsigned long long word = 0ull;
  const unsigned long long *src = t < nwords ? Q.row_pub + 3 * static_cast<size_t>(row_of(t / 3)) + t % 3 : nullptr;
  int polls = 0;
  bool timed_out = false;
  while (true) {
    if (t < nwords && word == 0ull) word = load_agent(src);
    if (__syncthreads_and(t >= nwords || word != 0ull)) break;
    if (++polls >= kMaxPolls) {
      timed_out = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (timed_out) {                                    // no chain without the statistics: nothing emitted
    if (t < kp1) P.out_tokens[static_cast<size_t>(b) * kp1 + t] = -1;
    if (t == 0) {
      P.accept_len[b] = 0;
      P.emit_count[b] = 0;
      if (P.emit_offsets) __hip_atomic_store(P.ecnt + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (P.final_mass) P.final_mass[b] = 0.0;
      if (P.status) P.status[b] = SPEC_ST_INCOMPLETE;
    }
    return;
  }
  if (t < nwords) unpack_stats(L.stat[t / 3], t % 3, word);
  __syncthreads();

  // ---- the tries and the chain
  if (t < k) {
    int2 r = make_int2(0, SPEC_ST_DRAFT_OOR);
    if (x_t >= 0 && x_t < V)
      r = try_draft(proc_prob(zp_t, L.stat[t], P.invT), proc_prob(zq_t, L.stat[kp1 + t], P.invT), u_t);
    sh_acc[t] = r.x;
    sh_st[t] = r.y;
    sh_d[t] = x_t;
  }
  __syncthreads();
  if (t == 0) sh_ch = fold_chain(k, rem, P.eos, sh_acc, sh_st, sh_d);
  __syncthreads();
  const int4 ch = sh_ch;
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
    const bool resid = mode == MODE_RESID;
    LogitRow<BF16> r;
    r.a = Src::prow(P, b, jrow);
    r.sa = L.stat[jrow];
    r.b = resid ? Src::qrow(P, b, jrow) : nullptr;
    if (resid) r.sb = L.stat[kp1 + jrow];
    r.invT = P.invT;
    r.resid = resid;
    // list lengths of the row drawn from (indexed, not through a pointer
    // that may point anywhere: LDS reads then wait for LDS only)
    auto cnt = [&](int q) { return pre ? L.cnt[jrow * nS + q] : L.cnt_row[q]; };
    if (!pre) {
      if (t < nS) L.cnt_row[t] = Q.list_cnt[static_cast<size_t>(b * kp1 + jrow) * nS + t];
    }
    // without top-k the lists hold every entry at or above their slice's cut
    // (and nothing below it), so they hold the kept entries when the row's
    // threshold reaches the largest cut
    const bool topk = Q.cfg.top_k > 0 && Q.cfg.top_k < V;
    if (!topk && t < kWave) {
      const uint32_t c = t < nS ? Q.list_cut[static_cast<size_t>(b * kp1 + jrow) * nS + t] : 0u;
      const uint32_t cm = wave_max_u(c);
      if (t == 0) sh_cutmax = cm;
    }
    if (t == 0) sh_n = 0;
    if (t < nS) L.qn[t] = 0;
    __syncthreads();
    bool complete = topk || r.sa.theta >= sh_cutmax;
    for (int q = 0; q < nS; ++q) complete = complete && cnt(q) <= cap;
    if (complete && r.sa.mass > 0.0) {
      // the kept entries of the row drawn from (wave w: lists w, w + 16, ...)
      for (int q = w; q < nS; q += kProcWaves) {
        const int c = cnt(q);
        const size_t seg = seg_of(jrow, q);
        for (int i0 = 0; i0 < c; i0 += kWave) {
          const int i = i0 + lane;
          bool keep = false;
          float z = 0.0f;
          int v = 0;
          if (i < c) {
            if (pre && i < kPfHead) {
              z = L.pf_val[(jrow * nS + q) * kPfHead + i];
              v = L.pf_idx[(jrow * nS + q) * kPfHead + i];
            } else {                  // (atomic loads, which the compiler does not merge with the
                                      // LDS reads above into generic ones; those would wait for
                                      // every outstanding global access)
              z = load_agent(Q.lists + seg + i);
              v = load_agent(Q.list_idx + seg + i);
            }
            keep = f32_order_key(z) >= r.sa.theta;
          }
          const int slot = wave_append(keep, &sh_n);
          if (keep && slot < kProcThreads) {
            L.idx[slot] = v;
            L.val[slot] = z;
            L.qs[slot] = q;
          }
          const int kq = __popcll(__ballot(keep));
          if (lane == 0 && kq > 0) atomicAdd(&L.qn[q], kq);
        }
      }
    }
    __syncthreads();
    const int n = sh_n;
    if (complete && n <= kProcThreads) {
      // order the n kept entries by index (distinct), one per lane
      if (t < n) L.ord[t] = -1;
      if (n <= kRankAll) {
        // few: each ranks itself among all of them
        if (t >= n && t < ((n + 3) & ~3)) L.idx[t] = INT_MAX;
        __syncthreads();
        if (t < n) {
          const int my = L.idx[t];
          const int4 *q4 = reinterpret_cast<const int4 *>(L.idx);
          int rank = 0;
          for (int i = 0; i < (n + 3) >> 2; ++i) {
            const int4 e = q4[i];
            rank += (e.x < my) + (e.y < my) + (e.z < my) + (e.w < my);
          }
          L.ord[rank] = my;
          L.ordv[rank] = L.val[t];
        }
      } else {
        // many: a slice's indices lie in one range, so the entries are
        // grouped by slice (offsets from the slices' counts) and ranked
        // within their slice
        if (t < kWave) {
          const int c = t < nS ? L.qn[t] : 0;
          const int x = wave_incl_scan(c) - c;
          if (t < nS) {
            L.qbase[t] = x;
            L.qpos[t] = 0;
          }
        }
        __syncthreads();
        if (t < n) {
          const int q = L.qs[t];
          const int pos = L.qbase[q] + atomicAdd(&L.qpos[q], 1);
          L.gidx[pos] = L.idx[t];
          L.gval[pos] = L.val[t];
          L.gq[pos] = q;
        }
        __syncthreads();
        if (t < n) {
          const int q = L.gq[t], b0 = L.qbase[q], nq = L.qn[q];
          const int my = L.gidx[t];
          int rank = 0;
          for (int i = 0; i < nq; ++i) rank += L.gidx[b0 + i] < my;
          L.ord[b0 + rank] = my;
          L.ordv[b0 + rank] = L.gval[t];
        }
      }
      __syncthreads();
      const int v = t < n ? L.ord[t] : -1;
      float pa = 0.0f, x = 0.0f;
      if (v >= 0 && v < V) {
        // a listed logit is the row's (a -0 comes back as +0, with the same
        // key and weight)
        pa = proc_prob(L.ordv[t], r.sa, r.invT);
        x = resid ? fmaxf(pa - proc_prob(logit_at<BF16>(r.b, v), r.sb, r.invT), 0.0f) : pa;
      }
      double incl = pv_incl_scan(static_cast<double>(x), sh_dw, &S);
      if (isfinite(S) && !(S > 0.0)) {
        st |= SPEC_ST_RESID_ZERO;
        if (resid) {                                  // fall back to the target row p'_j itself
          x = pa;
          incl = pv_incl_scan(static_cast<double>(x), sh_dw, &S);
        }
      }
      if (!isfinite(S)) {
        st |= SPEC_ST_NONFINITE;
        tok = 0;
      } else if (!(S > 0.0)) {
        tok = 0;
      } else {
        const double T = static_cast<double>(u_draw) * S;
        const int2 mm = pv_min_max(t < n && incl > T ? t : INT_MAX, t < n && x > 0.0f ? t : -1, sh_iw);
        tok = max(L.ord[mm.x != INT_MAX ? mm.x : mm.y], 0);
      }
    } else {
      tok = pv_draw_dense<BF16>(r, V, P.vec != 0, u_draw, S, st, L.cm, sh_dw, sh_iw);
    }
  }
  if (t < kp1) {                                      // accepted drafts, then the drawn token
    int val = -1;
    if (t < m) val = x_t;
    else if (t == m && mode != MODE_NONE) val = tok;
    P.out_tokens[static_cast<size_t>(b) * kp1 + t] = val;
  }
  if (t == 0) {
    if (P.final_mass) P.final_mass[b] = mode != MODE_NONE ? S : 0.0;
    if (P.status) P.status[b] = st;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kProcThreads) void proc_verify_kernel(ProcVerifyParams X) {
  // the statistics' histograms, or a finisher's staging
  __shared__ unsigned long long lh[256 * kWave];
  const int blk = blockIdx.x, rows = X.proc.rows;
  if (blk < rows) {
    const ProcStats st = proc_row_stats<BF16>(X.proc, blk, lh);
    if (threadIdx.x == 0) publish_stats(X.proc.row_pub + 3 * static_cast<size_t>(blk), st);
  } else if (blk < rows + X.smp.B) {
    pv_finish<BF16>(X, blk - rows, lh);
  } else {
    finish_offsets(X.smp);
  }
}

}  // namespace

// Launches the statistics kernel over rows [0, rows); shared with the
// stochastic verification from logits.
// Workspace after the row statistics: candidate lists, then the per-slice
// arrays, sized for the larger slice count (float32 slices of 8192 logits).
struct ProcWs {
  size_t lists, cnt, cut, lb, smax, smin, stot, total;
};
static ProcWs proc_ws_layout(int rows, int V) {
  const size_t R = static_cast<size_t>(rows);
  const size_t S = (static_cast<size_t>(V) + kSliceThreads * kSliceLoads * 4 - 1) / (kSliceThreads * kSliceLoads * 4);
  ProcWs L;
  L.lists = 0;
  L.cnt = L.lists + round_up(R * kCandCap * sizeof(float), 256);
  L.cut = L.cnt + round_up(R * S * sizeof(int), 256);
  L.lb = L.cut + round_up(R * S * sizeof(uint32_t), 256);
  L.smax = L.lb + round_up(R * S * sizeof(uint32_t), 256);
  L.smin = L.smax + round_up(R * S * sizeof(uint32_t), 256);
  L.stot = L.smin + round_up(R * S * sizeof(uint32_t), 256);
  L.total = L.stot + round_up(R * S * sizeof(unsigned long long), 256);
  return L;
}

size_t proc_list_bytes(int rows, int V) { return proc_ws_layout(rows, V).total; }

static ProcParams proc_params(const void *za, const void *zb, int rows_a, int rows, int V, bool bf16, Temper invT,
                              int top_k, float top_p, ProcStats *stats, float *probs) {
  ProcParams P;
  P.za = za;
  P.zb = zb;
  P.rows_a = rows_a;
  P.rows = rows;
  P.V = V;
  P.cfg.invT = invT;
  P.cfg.top_k = top_k;
  P.cfg.top_p = top_p;
  P.stats = stats;
  P.probs = probs;
  P.lists = nullptr;
  P.list_cnt = nullptr;
  P.list_cut = nullptr;
  P.list_lb = nullptr;
  P.list_idx = nullptr;
  P.row_pub = nullptr;
  P.lb_rank = 0;
  P.sl_max = P.sl_min = nullptr;
  P.sl_tot = nullptr;
  const int slice = kSliceThreads * kSliceLoads * (bf16 ? 8 : 4);
  P.S = (V + slice - 1) / slice;
  P.seg_cap = kCandCap / P.S;
  P.cut_rank = 0;
  return P;
}

// Top-k through the slice lists: K <= 256 (the cut is the K-th largest of a
// slice's 256 lane maxima) and lists of at most half a segment.
static bool topk_lists(const ProcParams &P, int top_k, int V) {
  return top_k > 0 && top_k < V && top_k <= kSliceThreads && top_k <= P.seg_cap / 2;
}

// The slice kernel, listing each slice at its rank-th largest lane maximum
// (bounds: also each slice's ceil(K / S)-th largest, for top-k).
static void launch_slices(ProcParams &P, const ProcWs &L, unsigned char *w, int rank, bool bounds, int top_k,
                          bool bf16, hipStream_t s) {
  P.lists = reinterpret_cast<float *>(w + L.lists);
  P.list_cnt = reinterpret_cast<int *>(w + L.cnt);
  P.list_cut = reinterpret_cast<uint32_t *>(w + L.cut);
  P.cut_rank = rank;
  if (bounds) {
    P.list_lb = reinterpret_cast<uint32_t *>(w + L.lb);
    P.lb_rank = (top_k + P.S - 1) / P.S;
  }
  const dim3 g(static_cast<unsigned>(P.rows * P.S)), blk(kSliceThreads);
  if (bf16)
    hipLaunchKernelGGL(proc_slice_kernel<true>, g, blk, 0, s, P);
  else
    hipLaunchKernelGGL(proc_slice_kernel<false>, g, blk, 0, s, P);
}

int launch_proc_stats(const void *za, const void *zb, int rows_a, int rows, int V, bool bf16,
                      Temper invT, int top_k, float top_p, ProcStats *stats, float *probs,
                      void *list_ws, hipStream_t s) {
  ProcParams P = proc_params(za, zb, rows_a, rows, V, bf16, invT, top_k, top_p, stats, probs);
  if (list_ws) {
    const ProcWs L = proc_ws_layout(rows, V);
    unsigned char *w = static_cast<unsigned char *>(list_ws);
    const dim3 g(static_cast<unsigned>(rows * P.S)), blk(kSliceThreads);
    if (top_k > 0 && top_k < V) {
      if (topk_lists(P, top_k, V)) launch_slices(P, L, w, top_k, true, top_k, bf16, s);
    } else {
      // no top-k: slice maxima (with top-p: the lists cut at the kToppRank-th
      // largest lane maximum, which also give them), then slice weights and
      // minima
      P.sl_max = reinterpret_cast<uint32_t *>(w + L.smax);
      P.sl_min = reinterpret_cast<uint32_t *>(w + L.smin);
      P.sl_tot = reinterpret_cast<unsigned long long *>(w + L.stot);
      if (top_p < 1.0f && kToppRank <= P.seg_cap / 2) {
        launch_slices(P, L, w, kToppRank, false, top_k, bf16, s);
      } else if (bf16) {
        hipLaunchKernelGGL(proc_slrange_kernel<true>, g, blk, 0, s, P);
      } else {
        hipLaunchKernelGGL(proc_slrange_kernel<false>, g, blk, 0, s, P);
      }
      if (bf16)
        hipLaunchKernelGGL(proc_slmass_kernel<true>, g, blk, 0, s, P);
      else
        hipLaunchKernelGGL(proc_slmass_kernel<false>, g, blk, 0, s, P);
    }
  }
  if (bf16)
    hipLaunchKernelGGL(proc_stats_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(kProcThreads), 0, s, P);
  else
    hipLaunchKernelGGL(proc_stats_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(kProcThreads), 0, s, P);
  return 0;
}

size_t proc_list_idx_bytes(int rows) { return round_up(static_cast<size_t>(rows) * kCandCap * sizeof(int32_t), 256); }

bool launch_sample_logits_lists(const SampleParams &S, bool bf16, int top_k, float top_p, ProcStats *stats,
                                void *list_ws, int32_t *list_idx, unsigned long long *row_pub, hipStream_t s) {
  const int rows_a = S.B * (S.k + 1), rows = S.B * (2 * S.k + 1);
  ProcVerifyParams X;
  X.proc = proc_params(S.zp, S.zq, rows_a, rows, S.V, bf16, S.invT, top_k, top_p, stats, nullptr);
  X.proc.list_idx = list_idx;
  X.proc.row_pub = row_pub;
  const ProcWs L = proc_ws_layout(rows, S.V);
  unsigned char *w = static_cast<unsigned char *>(list_ws);
  if (top_k > 0 && top_k < S.V) {
    if (!topk_lists(X.proc, top_k, S.V)) return false;
    launch_slices(X.proc, L, w, top_k, true, top_k, bf16, s);
  } else if (top_p < 1.0f && kToppRank <= X.proc.seg_cap / 2) {
    // top-p alone: lists at the kToppRank-th lane maximum, then the slices'
    // exact weights (the statistics' union check needs the row's total)
    X.proc.sl_max = reinterpret_cast<uint32_t *>(w + L.smax);
    X.proc.sl_min = reinterpret_cast<uint32_t *>(w + L.smin);
    X.proc.sl_tot = reinterpret_cast<unsigned long long *>(w + L.stot);
    launch_slices(X.proc, L, w, kToppRank, false, top_k, bf16, s);
    const dim3 gs(static_cast<unsigned>(rows * X.proc.S)), bs(kSliceThreads);
    if (bf16)
      hipLaunchKernelGGL(proc_slmass_kernel<true>, gs, bs, 0, s, X.proc);
    else
      hipLaunchKernelGGL(proc_slmass_kernel<false>, gs, bs, 0, s, X.proc);
  } else {
    return false;
  }
  X.smp = S;
  const dim3 g(static_cast<unsigned>(rows + S.B + (S.emit_offsets ? 1 : 0))), blk(kProcThreads);
  if (bf16)
    hipLaunchKernelGGL(proc_verify_kernel<true>, g, blk, 0, s, X);
  else
    hipLaunchKernelGGL(proc_verify_kernel<false>, g, blk, 0, s, X);
  return true;
}

bool proc_args_ok(float T, int top_k, float top_p, int V) {
  return T > 0.0f && T < INFINITY && top_k >= 0 && top_p > 0.0f && top_p <= 1.0f &&
         V >= 1 && V <= SPEC_PROC_MAX_V;
}

}  // namespace specv

using namespace specv;

extern "C" size_t spec_process_workspace_bytes(int R, int V) {
  if (R < 1 || V < 1 || V > SPEC_PROC_MAX_V) return 0;
  return round_up(static_cast<size_t>(R) * sizeof(ProcStats), 256) + proc_list_bytes(R, V);
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
  const size_t need = spec_process_workspace_bytes(R, V);
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
  void *lists = static_cast<unsigned char *>(ws) + round_up(static_cast<size_t>(R) * sizeof(ProcStats), 256);
  (void)hipGetLastError();
  launch_proc_stats(logits, logits, R, R, V, dt == SPEC_BF16, make_temper(temperature), top_k, top_p, stats,
                    probs, lists, s);
  if (row_max || row_threshold || row_mass)
    hipLaunchKernelGGL(proc_export_kernel, dim3((R + 255) / 256), dim3(256), 0, s, stats, R, row_max,
                       row_threshold, row_mass);
  return launch_status();
}
