// Same-length grouping of a window of ragged sequences (gfx950).
//
// The "Correctness Forensics for Batch Speculative Decoding" summary, 3.2,
// describes EXSPEC: sequences stay ragged and batches are formed from
// sequences of identical length found in a window larger than the batch
// size, with unpad-append-repad as the fallback.  The scheduler's algorithm
// body (App. C) is not on the page; the rule implemented here is stated in
// include/spec_verify.h.
//
// Design.  The window is small (<= SPEC_GROUP_MAX_N), so one workgroup (one
// lane per key up to 1024 keys, at least one wave) does it all: a bitonic
// sort of 64-bit keys (length in the high word,
// order-corrected for sign; window index in the low word), which makes every
// key distinct and the sort stable by construction (up to 1024 keys one per
// lane, strides below a wave by lane shuffles; larger windows in LDS); then
// run detection and two block-wide scans give each sorted position its run
// and the run's offsets among same-length members, same-length batches and
// fallback members (three 21-bit counts packed in one 64-bit scan), and every
// position writes its own output slots.  The work is latency-bound
// (microseconds); there is nothing to stream.
#include "common.h"

namespace specv {
namespace {

constexpr int kMaxThreads = 1024;

// Workgroup size for a window of P2 (a power of two) keys: one key per lane
// up to 1024 keys, at least one wave.  Smaller windows run on fewer waves, so
// every barrier and every lane-shuffle stage involves fewer waves.
inline int group_threads(int P2) { return P2 < kWave ? kWave : (P2 < kMaxThreads ? P2 : kMaxThreads); }

// Block-wide exclusive sum of one 64-bit value per lane (lane order); `sh`
// holds kThreads / kWave + 1 words; *total receives the block total.
// Barriers: call from every lane.
template <int kThreads>
__device__ inline unsigned long long block_excl_scan_u64(unsigned long long v, unsigned long long *sh,
                                                         unsigned long long *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  constexpr int nw = kThreads / kWave;
  const unsigned long long inc = wave_incl_scan(v);
  if (lane == kWave - 1) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    const unsigned long long x = lane < nw ? sh[lane] : 0ull;
    const unsigned long long xi = wave_incl_scan(x);
    if (lane < nw) sh[lane] = xi - x;
    if (lane == nw - 1) sh[nw] = xi;
  }
  __syncthreads();
  const unsigned long long r = inc - v + sh[w];
  *total = sh[nw];
  __syncthreads();
  return r;
}

template <int kThreads>
__global__ __launch_bounds__(kThreads) void group_kernel(const int32_t *lengths, int N, int B, int mg,
                                                          int P2, int32_t *perm, int32_t *batch_start,
                                                          int32_t *batch_len, int32_t *num_batches,
                                                          int32_t *num_grouped) {
  // sorted positions per lane: one below 1024 lanes (then N <= P2 <= kThreads)
  constexpr int kPer = kThreads < kMaxThreads ? 1 : SPEC_GROUP_MAX_N / kMaxThreads;
  extern __shared__ unsigned long long smem[];
  unsigned long long *keys = smem;                                  // [P2]
  int *run_start = reinterpret_cast<int *>(smem + P2);              // [N + 1]
  __shared__ int sh[kThreads / kWave + 1];
  __shared__ unsigned long long sh64[kThreads / kWave + 1];
  const int t = threadIdx.x;

  if (N == 0) {
    if (t == 0) {
      batch_start[0] = 0;
      *num_batches = 0;
      *num_grouped = 0;
    }
    return;
  }
  auto key_of = [&](int i) {
    return i < N ? (static_cast<unsigned long long>(static_cast<uint32_t>(lengths[i]) ^ 0x80000000u) << 32) |
                       static_cast<uint32_t>(i)
                 : ~0ull;
  };
  if (P2 <= kThreads) {
    // one key per lane: strides below a wave by lane shuffles, the others
    // through LDS (lanes past P2 hold padding and pair among themselves)
    unsigned long long v = key_of(t);
    for (int size = 2; size <= P2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        unsigned long long o = v;
        if (stride >= kWave) {
          if (t < P2) keys[t] = v;
          __syncthreads();
          if (t < P2) o = keys[t ^ stride];
          __syncthreads();
        } else {
          o = __shfl_xor(v, stride, kWave);
        }
        const bool lower = (t & stride) == 0, up = (t & size) == 0;
        v = (lower == up) ? (o < v ? o : v) : (o > v ? o : v);
      }
    }
    if (t < P2) keys[t] = v;
  } else {
    for (int i = t; i < P2; i += kThreads) keys[i] = key_of(i);
    __syncthreads();
    for (int size = 2; size <= P2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = t; i < P2 / 2; i += kThreads) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const unsigned long long a = keys[lo], c = keys[hi];
          if ((a > c) == up) {
            keys[lo] = c;
            keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();

  // lane t owns sorted positions [t*per, t*per + per) within [0, N)
  const int per = (N + kThreads - 1) / kThreads;
  const int p0 = min(N, t * per), p1 = min(N, p0 + per);
  int len[kPer], idx[kPer], start[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pos = p0 + i;
    if (pos < p1) {
      const unsigned long long kk = keys[pos];
      len[i] = static_cast<int>(static_cast<uint32_t>(kk >> 32) ^ 0x80000000u);
      idx[i] = static_cast<int>(static_cast<uint32_t>(kk));
      const int prev = pos > 0 ? static_cast<int>(static_cast<uint32_t>(keys[pos - 1] >> 32) ^ 0x80000000u) : 0;
      start[i] = (pos == 0 || prev != len[i]) ? 1 : 0;
    } else {
      len[i] = idx[i] = start[i] = 0;
    }
  }
  // run ids
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) cnt += start[i];
  int runs;
  int rid = block_excl_scan(cnt, sh, &runs) - 1;
  int run_of[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    rid += start[i];
    run_of[i] = rid;
    if (p0 + i < p1 && start[i]) run_start[rid] = p0 + i;
  }
  if (t == 0) run_start[runs] = N;
  __syncthreads();

  // per-run counts, placed at the run's first position
  int nu[kPer], nb[kPer], nf[kPer], off[kPer];
  int su = 0, sb = 0, sf = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    nu[i] = nb[i] = nf[i] = 0;
    off[i] = 0;
    if (p0 + i < p1) {
      const int s = run_start[run_of[i]], e = run_start[run_of[i] + 1];
      const int c = e - s, full = c / B, rem = c - full * B;
      nu[i] = full * B + (rem >= mg ? rem : 0);
      nb[i] = full + (rem >= mg && rem > 0 ? 1 : 0);
      nf[i] = c - nu[i];
      off[i] = p0 + i - s;
      if (start[i]) {
        su += nu[i];
        sb += nb[i];
        sf += nf[i];
      }
    }
  }
  // the three counts scanned at once: 21-bit fields of one 64-bit word (every
  // sum is at most N <= SPEC_GROUP_MAX_N < 2^21, so no field carries over)
  static_assert(SPEC_GROUP_MAX_N < (1 << 21), "21-bit count fields");
  int TU, TB, TF, xu, xb, xf;
  {
    const unsigned long long packed = (static_cast<unsigned long long>(su) << 42) |
                                      (static_cast<unsigned long long>(sb) << 21) | static_cast<unsigned long long>(sf);
    unsigned long long tot;
    const unsigned long long ex = block_excl_scan_u64<kThreads>(packed, sh64, &tot);
    constexpr unsigned long long m21 = (1ull << 21) - 1;
    xu = static_cast<int>(ex >> 42);
    xb = static_cast<int>((ex >> 21) & m21);
    xf = static_cast<int>(ex & m21);
    TU = static_cast<int>(tot >> 42);
    TB = static_cast<int>((tot >> 21) & m21);
    TF = static_cast<int>(tot & m21);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (p0 + i >= p1) continue;
    // offsets of this position's run: the running exclusive sums hold every
    // earlier run, plus this run itself unless it starts at this position
    const int ou = start[i] ? xu : xu - nu[i];
    const int ob = start[i] ? xb : xb - nb[i];
    const int of = start[i] ? xf : xf - nf[i];
    const int o = off[i];
    if (o < nu[i]) {
      perm[ou + o] = idx[i];
      if (o % B == 0) {
        batch_start[ob + o / B] = ou + o;
        batch_len[ob + o / B] = len[i];
      }
    } else {
      const int f = of + (o - nu[i]);
      perm[TU + f] = idx[i];
      if (f % B == 0) {
        batch_start[TB + f / B] = TU + f;
        batch_len[TB + f / B] = -1;
      }
    }
    if (start[i]) {
      xu += nu[i];
      xb += nb[i];
      xf += nf[i];
    }
  }
  if (t == 0) {
    const int nbat = TB + (TF + B - 1) / B;
    batch_start[nbat] = N;
    *num_batches = nbat;
    *num_grouped = TU;
  }
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" int spec_group_same_length(const int32_t *lengths, int N, int B, int min_group, int32_t *perm,
                                      int32_t *batch_start, int32_t *batch_len, int32_t *num_batches,
                                      int32_t *num_grouped, spec_stream_t stream) {
  if (!batch_start || !num_batches || !num_grouped) return SPEC_EINVAL;
  if (N > 0 && (!lengths || !perm || !batch_len)) return SPEC_EINVAL;
  if (N < 0 || B < 1 || min_group < 1) return SPEC_EINVAL;
  if (N > SPEC_GROUP_MAX_N) return SPEC_ECAPACITY;
  const size_t n4 = static_cast<size_t>(N) * 4;
  const void *outs[] = {perm, batch_start, batch_len, num_batches, num_grouped};
  const size_t out_n[] = {n4, n4 + 4, n4, 4, 4};
  for (int i = 0; i < 5; ++i) {
    if (overlaps(outs[i], out_n[i], lengths, n4)) return SPEC_EINVAL;
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }
  int P2 = 2;
  while (P2 < N) P2 <<= 1;
  const size_t shmem = static_cast<size_t>(P2) * 8 + static_cast<size_t>(N + 1) * 4;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  switch (group_threads(P2)) {
#define SPEC_GROUP_LAUNCH(NT)                                                                                   \
  case NT:                                                                                                      \
    hipLaunchKernelGGL(group_kernel<NT>, dim3(1), dim3(NT), shmem, s, lengths, N, B, min_group, P2, perm,      \
                       batch_start, batch_len, num_batches, num_grouped);                                       \
    break;
    SPEC_GROUP_LAUNCH(64)
    SPEC_GROUP_LAUNCH(128)
    SPEC_GROUP_LAUNCH(256)
    SPEC_GROUP_LAUNCH(512)
    SPEC_GROUP_LAUNCH(1024)
#undef SPEC_GROUP_LAUNCH
    default:
      return SPEC_EINVAL;
  }
  return launch_status();
}
