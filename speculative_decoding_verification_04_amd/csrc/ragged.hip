// Unpad-append-repad between ragged per-sequence caches and a left-padded
// rectangle (gfx950).
//
// The "Correctness Forensics for Batch Speculative Decoding" summary, 3.2:
// EXSPEC keeps sequences ragged and batches sequences of one length, which
// need no realignment; when no same-length group forms, it falls back to
// unpad-append-repad.  Here the ragged caches are one pool
// [L][2][N][H][Cs][D] in which sequence s holds its n_s rows at columns
// [0, n_s) of each (layer, K/V, head) plane.  A mixed batch of B pool
// sequences is copied into a rectangle [L][2][B][H][C][D] right-aligned at
// column E (repad); after the verify forward wrote its k+1 slots at
// [E, E + k + 1) and the verify call gave e_i, each member's rows
// [E - n_i, E + e_i) -- its cached rows and its kept slots -- are copied back
// to columns [0, n_i + e_i) of its pool plane (unpad and append).
//
// Design.  Both are plain copies between two buffers, bound by HBM bandwidth
// (read + write of every copied byte).  One 256-lane workgroup per (layer,
// K/V, member, head) plane copies that plane's contiguous run of rows with
// 16-byte non-temporal loads and stores, four in flight per lane; the member's
// state (pool index, lengths, E) is read once per workgroup.
#include "common.h"

namespace specv {
namespace {

constexpr int kThreads = 256;
constexpr int kU = 4;

struct RaggedParams {
  const unsigned char *src;
  unsigned char *dst;
  int L, N, H, Cs, D, B, C, elt;
  long long row_bytes;           // D * elt
  const int32_t *index, *kv_len, *emit_count, *end_col;
  int32_t *kv_len_out, *status;
  bool unpad;
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

template <int VB>
struct Word;
template <> struct Word<16> { using T = v4u; };
template <> struct Word<8> { using T = v2u; };
template <> struct Word<4> { using T = uint32_t; };
template <> struct Word<2> { using T = uint16_t; };

// Status of member i (0 = valid): the pool index, lengths and E must describe
// ranges inside both buffers.
__device__ inline int member_status(const RaggedParams &P, int i, int E) {
  if (E < 0 || E > P.C) return SPEC_ST_CAPACITY;
  const int s = P.index[i], n = P.kv_len[i];
  const int e = P.unpad ? P.emit_count[i] : 0;
  if (s < 0 || s >= P.N || n < 0 || n > E || e < 0 || E + e > P.C || n + e > P.Cs) return SPEC_ST_BAD_STATE;
  return 0;
}

template <int VB>
__global__ __launch_bounds__(kThreads) void ragged_copy_kernel(RaggedParams P) {
  using T = typename Word<VB>::T;
  const int plane = blockIdx.x;                        // ((l * 2 + kv) * B + i) * H + h
  const int h = plane % P.H;
  const int i = (plane / P.H) % P.B;
  const int lkv = plane / (P.H * P.B);                 // l * 2 + kv
  const int E = *P.end_col;
  const int st = member_status(P, i, E);
  if (h == 0 && lkv == 0 && threadIdx.x == 0) {
    if (P.status) P.status[i] = st;
    if (P.kv_len_out) P.kv_len_out[i] = st ? P.kv_len[i] : P.kv_len[i] + P.emit_count[i];
  }
  if (st) return;
  const int s = P.index[i], n = P.kv_len[i];
  const int rows = P.unpad ? n + P.emit_count[i] : n;
  const long long pool_plane = ((static_cast<long long>(lkv) * P.N + s) * P.H + h) * P.Cs;
  const long long rect_plane = ((static_cast<long long>(lkv) * P.B + i) * P.H + h) * P.C;
  // pool rows [0, rows) <-> rectangle rows [E - n, E - n + rows)
  const long long pool_off = pool_plane * P.row_bytes;
  const long long rect_off = (rect_plane + (E - n)) * P.row_bytes;
  const T *src = reinterpret_cast<const T *>(P.src + (P.unpad ? rect_off : pool_off));
  T *dst = reinterpret_cast<T *>(P.dst + (P.unpad ? pool_off : rect_off));
  const long long nw = rows * P.row_bytes / VB;
  if (nw <= 0) return;
  // Every lane issues every load and store (no per-lane branches), so the wait
  // for one step's loads leaves the next step's loads and the previous step's
  // stores in flight; indices past the run are clamped to its last vector,
  // which such lanes copy again (the same value to the same cell).  Three
  // register buffers rotate, so none is reloaded right after its stores.
  const long long last = nw - 1;
  const int t = threadIdx.x;
  constexpr long long kStep = static_cast<long long>(kThreads) * kU;
  long long w0 = 0;
  T b0[kU], b1[kU], b2[kU];
  auto load = [&](T (&x)[kU], long long base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) x[u] = __builtin_nontemporal_load(src + min(base + u * kThreads + t, last));
  };
  auto step = [&](T (&cur)[kU], T (&nxt)[kU]) __attribute__((always_inline)) {
    const long long nb = w0 + kStep;
    load(nxt, nb);
#pragma unroll
    for (int u = 0; u < kU; ++u) __builtin_nontemporal_store(cur[u], dst + min(w0 + u * kThreads + t, last));
    w0 = nb;
    return nb < nw;
  };
  load(b0, 0);
  while (step(b0, b1) && step(b1, b2) && step(b2, b0)) {
  }
}

int ragged_launch(RaggedParams P, const void *pool, const void *rect, hipStream_t s) {
  const long long planes = static_cast<long long>(P.L) * 2 * P.B * P.H;
  if (planes >= INT32_MAX) return SPEC_EINVAL;
  int vb = 2;
  for (int c : {16, 8, 4}) {
    if (P.row_bytes % c == 0 && aligned(pool, c) && aligned(rect, c)) { vb = c; break; }
  }
  if (P.elt == 4 && vb < 4) return SPEC_EINVAL;
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(planes));
  switch (vb) {
    case 16: hipLaunchKernelGGL(ragged_copy_kernel<16>, grid, dim3(kThreads), 0, s, P); break;
    case 8: hipLaunchKernelGGL(ragged_copy_kernel<8>, grid, dim3(kThreads), 0, s, P); break;
    case 4: hipLaunchKernelGGL(ragged_copy_kernel<4>, grid, dim3(kThreads), 0, s, P); break;
    default: hipLaunchKernelGGL(ragged_copy_kernel<2>, grid, dim3(kThreads), 0, s, P); break;
  }
  return launch_status();
}

int ragged_call(const void *pool, const void *rect, spec_dtype dt, int L, int N, int H, int Cs, int D, int B,
                int C, const int32_t *index, const int32_t *kv_len, const int32_t *emit_count,
                const int32_t *end_col, int32_t *kv_len_out, int32_t *status, bool unpad, spec_stream_t stream) {
  if (!pool || !rect || !index || !kv_len || !end_col) return SPEC_EINVAL;
  if (unpad && (!emit_count || !kv_len_out)) return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (L < 1 || N < 1 || H < 1 || Cs < 1 || D < 1 || B < 1 || C < 1) return SPEC_EINVAL;
  const int elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(pool, elt) || !aligned(rect, elt)) return SPEC_EINVAL;
  const size_t row = static_cast<size_t>(D) * elt;
  const size_t pool_n = static_cast<size_t>(L) * 2 * N * H * Cs * row;
  const size_t rect_n = static_cast<size_t>(L) * 2 * B * H * C * row;
  const size_t b4 = static_cast<size_t>(B) * 4;
  const void *ins[] = {index, kv_len, emit_count, end_col, unpad ? rect : pool};
  const size_t in_n[] = {b4, b4, unpad ? b4 : 0, 4, unpad ? rect_n : pool_n};
  const void *outs[] = {unpad ? pool : rect, kv_len_out, status};
  const size_t out_n[] = {unpad ? pool_n : rect_n, b4, b4};
  for (int o = 0; o < 3; ++o) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[o], out_n[o], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = o + 1; j < 3; ++j)
      if (overlaps(outs[o], out_n[o], outs[j], out_n[j])) return SPEC_EINVAL;
  }
  RaggedParams P;
  P.src = static_cast<const unsigned char *>(unpad ? rect : pool);
  P.dst = static_cast<unsigned char *>(const_cast<void *>(unpad ? pool : rect));
  P.L = L;
  P.N = N;
  P.H = H;
  P.Cs = Cs;
  P.D = D;
  P.B = B;
  P.C = C;
  P.elt = elt;
  P.row_bytes = static_cast<long long>(row);
  P.index = index;
  P.kv_len = kv_len;
  P.emit_count = emit_count;
  P.end_col = end_col;
  P.kv_len_out = kv_len_out;
  P.status = status;
  P.unpad = unpad;
  return ragged_launch(P, pool, rect, static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" int spec_repad_kv(const void *pool, void *rect, spec_dtype dt, int L, int N, int H, int Cs, int D,
                             int B, int C, const int32_t *index, const int32_t *kv_len, const int32_t *end_col,
                             int32_t *status, spec_stream_t stream) {
  return ragged_call(pool, rect, dt, L, N, H, Cs, D, B, C, index, kv_len, nullptr, end_col, nullptr, status, false,
                     stream);
}

extern "C" int spec_unpad_kv(const void *rect, void *pool, spec_dtype dt, int L, int N, int H, int Cs, int D,
                             int B, int C, const int32_t *index, const int32_t *kv_len, const int32_t *emit_count,
                             const int32_t *end_col, int32_t *kv_len_out, int32_t *status, spec_stream_t stream) {
  return ragged_call(pool, rect, dt, L, N, H, Cs, D, B, C, index, kv_len, emit_count, end_col, kv_len_out, status,
                     true, stream);
}
