// Greedy verification of a batch of speculative rounds (gfx950).
//
// What it computes follows the greedy commitment of the zero-to-sglang
// "Chapter 10 Speculative Decoding (Code Walkthrough)" 4.1 and the BatchVerify
// description in the "Correctness Forensics for Batch Speculative Decoding"
// summary, App. D; the row alignment (row j verifies draft j, row k is the
// bonus row) is the walkthrough's 3.3 table.
//
// Design.  The logits are the only large input (B*(k+1)*V elements), so the
// kernel is one streaming pass over them, bound by HBM bandwidth.  Each row is
// cut into chunks of kThreads*VEC*U elements; one workgroup per (row, chunk)
// loads its chunk with 16-byte loads (U loads in flight per lane), takes the
// chunk maximum with plain max instructions, and then looks up the first
// index holding that maximum only in the lanes that hold it.  The chunk result
// is packed into a 64-bit key (value order high, UINT32_MAX - index low) so
// that the maximum key is the row argmax with the lowest-index tie rule.
// The last workgroup of a sequence to finish (agent-scope ticket counter)
// reduces its (k+1)*chunks keys, walks the drafts and writes the sequence's
// outputs; the last sequence to finish writes the emit offsets.  Keys and
// counters are zeroed by the workgroup that consumes them, so the whole
// workspace is zero again when the kernel ends (and can be reused for any
// shape).
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
  uint32_t *seq_ctr;  // [B]
  uint32_t *done_ctr; // [1]
};

struct GreedyWs {
  size_t keys, seq, done, total;
};

inline GreedyWs greedy_ws_layout(int B, int k, int chunks) {
  GreedyWs w;
  w.keys = 0;
  w.seq = round_up(static_cast<size_t>(B) * (k + 1) * chunks * sizeof(uint64_t), 256);
  w.done = w.seq + round_up(static_cast<size_t>(B) * sizeof(uint32_t), 256);
  w.total = w.done + 256;
  return w;
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

// Position (0..VEC-1) of the first element equal to m, or -1.
template <bool BF16>
__device__ inline int vec_find(uint4 x, float m) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (lo_bf16(w[i]) == m) return 2 * i;
      if (hi_bf16(w[i]) == m) return 2 * i + 1;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (__uint_as_float(w[i]) == m) return i;
  }
  return -1;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void greedy_verify_kernel(GreedyParams P) {
  using Tr = GreedyTraits<BF16>;
  constexpr int ELT = Tr::ELT, VEC = Tr::VEC, U = Tr::U;
  __shared__ float sh_max[kWaves];
  __shared__ int sh_idx[kWaves];
  __shared__ unsigned long long sh_row[SPEC_MAX_K + 1];
  __shared__ int sh_flag;
  __shared__ int sh_scan[kWaves + 1];

  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int row = blockIdx.x / P.chunks;
  const int c = blockIdx.x - row * P.chunks;
  const int kp1 = P.k + 1;
  const int b = row / kp1;
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
    buf[u] = vi < nv ? *reinterpret_cast<const uint4 *>(rowp + static_cast<size_t>(s + vi * VEC) * ELT)
                     : neg_inf_vec<BF16>();
  }
  if (has_tail) tv = load_elem<BF16>(rowp, s + nv * VEC + t);

  float lmax = fmaxf(hv, tv);
#pragma unroll
  for (int u = 0; u < U; ++u) lmax = fmaxf(lmax, vec_max<BF16>(buf[u]));

  const float wm = wave_max(lmax);
  if (lane == 0) sh_max[w] = wm;
  __syncthreads();
  float bmax = sh_max[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) bmax = fmaxf(bmax, sh_max[i]);

  // First index of the chunk maximum: only lanes holding it search; each
  // lane's elements are visited in increasing index order.
  int cand = INT_MAX;
  if (lmax == bmax) {
    if (has_head && hv == bmax) {
      cand = t;
    } else {
      bool found = false;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vi = t + u * kThreads;
        if (!found && vi < nv) {
          const int q = vec_find<BF16>(buf[u], bmax);
          if (q >= 0) {
            cand = s + vi * VEC + q;
            found = true;
          }
        }
      }
      if (!found && has_tail && tv == bmax) cand = s + nv * VEC + t;
    }
  }
  const int wc = wave_min(cand);
  if (lane == 0) sh_idx[w] = wc;
  __syncthreads();
  if (t == 0) {
    int bi = sh_idx[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) bi = min(bi, sh_idx[i]);
    const uint64_t key = bi == INT_MAX ? 0ull : argmax_key(bmax, bi);
    store_agent(&P.keys[static_cast<size_t>(row) * P.chunks + c], key);
    const uint32_t prev = ticket_agent(&P.seq_ctr[b]);
    sh_flag = prev == static_cast<uint32_t>(kp1 * P.chunks) - 1u;
  }
  __syncthreads();
  if (!sh_flag) return;

  // ---- last workgroup of sequence b: row argmaxes and the commit walk ----
  acquire_agent();
  for (int i = t; i < kp1; i += kThreads) sh_row[i] = 0ull;
  __syncthreads();
  const int nkeys = kp1 * P.chunks;
  const uint64_t *kb = P.keys + static_cast<size_t>(b) * nkeys;
  for (int i = t; i < nkeys; i += kThreads) {
    atomicMax(&sh_row[i / P.chunks], static_cast<unsigned long long>(load_agent(kb + i)));
    store_agent(const_cast<uint64_t *>(kb) + i, static_cast<uint64_t>(0));   // leave the workspace zeroed
  }
  __syncthreads();
  if (t == 0) {
    store_agent(&P.seq_ctr[b], 0u);
    const int32_t *d = P.draft + static_cast<size_t>(b) * P.k;
    int32_t *out = P.out_tokens + static_cast<size_t>(b) * kp1;
    const int rem = P.remaining ? P.remaining[b] : -1;   // negative: no budget
    int st = 0;
    for (int j = 0; j < P.k; ++j)
      if (d[j] < 0 || d[j] >= P.V) st |= SPEC_ST_DRAFT_OOR;
    int cnt = 0, acc = 0;
    if (rem != 0) {
      bool stop = false;
      for (int j = 0; j < P.k && !stop; ++j) {
        const int tj = argmax_key_index(sh_row[j]);
        out[cnt++] = tj;
        const bool match = tj == d[j];
        acc += match;
        if ((P.eos >= 0 && tj == P.eos) || cnt == rem || !match) stop = true;
      }
      if (!stop) out[cnt++] = argmax_key_index(sh_row[P.k]);
    }
    for (int i = cnt; i < kp1; ++i) out[i] = -1;
    P.accept_len[b] = acc;
    if (P.status) P.status[b] = st;
    store_agent(&P.emit_count[b], cnt);
    const uint32_t prev = ticket_agent(P.done_ctr);
    sh_flag = prev == static_cast<uint32_t>(P.B) - 1u;
  }
  __syncthreads();
  if (!sh_flag) return;

  // ---- last sequence: emit offsets ----
  acquire_agent();
  if (P.emit_offsets) block_offsets(P.emit_count, P.emit_offsets, P.B, sh_scan);
  if (t == 0) store_agent(P.done_ctr, 0u);
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_greedy_workspace_bytes(int B, int k, int V, spec_dtype dt) {
  if (B < 1 || k < 1 || V < 1 || k > SPEC_MAX_K) return 0;
  return greedy_ws_layout(B, k, greedy_chunks(V, dt)).total;
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
  const GreedyWs lay = greedy_ws_layout(B, k, chunks);
  if (ws_bytes < lay.total || !aligned(ws, 256)) return SPEC_EWORKSPACE;

  const size_t nl = static_cast<size_t>(B) * (k + 1) * V * elt;
  const void *ins[] = {logits, draft, remaining, ws};
  const size_t in_n[] = {nl, static_cast<size_t>(B) * k * 4, static_cast<size_t>(B) * 4, lay.total};
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
  unsigned char *wb = static_cast<unsigned char *>(ws);
  P.keys = reinterpret_cast<uint64_t *>(wb + lay.keys);
  P.seq_ctr = reinterpret_cast<uint32_t *>(wb + lay.seq);
  P.done_ctr = reinterpret_cast<uint32_t *>(wb + lay.done);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dt == SPEC_BF16)
    hipLaunchKernelGGL(greedy_verify_kernel<true>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL(greedy_verify_kernel<false>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s, P);
  return launch_status();
}
