// Commit: in-place realignment of the contiguous left-padded KV rectangle,
// position ids and attention mask (gfx950).
//
// What it computes is the unpad-append-repad realignment of the
// "Correctness Forensics for Batch Speculative Decoding" summary (sections 3.1
// and App. B): keep each sequence's cached rows plus the first e_b verify
// slots (the last emitted token has no KV yet: App. D, and the zero-to-sglang
// walkthrough 5.2), right-align every sequence to E' = E + max_b e_b, and
// rebuild position ids from the mask.
//
// Design.  The move is a right shift of a contiguous column range by
// delta_b = M - e_b columns inside each (layer, K/V, sequence, head) plane of
// C x D elements; sequences with delta_b = 0 do not move and cost nothing.
// It is a pure copy bound by HBM bandwidth (read + write of every moved byte).
//   * One workgroup per moving plane.  The moved bytes form one contiguous
//     range; the workgroup walks it from the right end to the left in tiles of
//     kThreads * kTileVec 16-byte vectors (112 KB for the wide walker),
//     consecutive lanes on consecutive vectors, with non-temporal loads and
//     stores (every byte is touched once).
//   * In-place overlap: a tile is loaded into registers, every lane waits for
//     its loads to land, a workgroup barrier follows, and only then is the
//     tile stored delta columns to the right.  The tile to its left is loaded
//     before that store: its source ends delta columns before this tile's
//     destination begins, so the two never overlap; and a tile's destination
//     only overlaps its own source and the source of the tile to its right,
//     both already in registers.
//   * Few, wide walkers: each workgroup reserves more than half of a CU's LDS,
//     so one runs per CU and about one plane per CU is in flight.  Planes are
//     dispatched in address order, so the planes in flight sit in one window
//     of memory.  Many narrow walkers (several per CU, each on its own plane
//     far from the others) keep more DRAM pages open at once and measured
//     about 10% slower on MI355X; so did longest-move-first dispatch.
//   * Planes smaller than one wide tile take narrow walkers instead (256
//     lanes, 16 KB tiles, no reservation, several per CU): there a wide tile
//     leaves most lanes idle and one plane per CU leaves the memory system
//     idle between planes (a draft cache of 64-token prefixes re-synced 3x
//     faster).  Planes of up to 512 KB take two 512-lane walkers per CU
//     (56 KB tiles): a CU then alternates between two planes of a few tiles
//     each (0.60 -> 0.65 of peak for planes of 119 KB, 0.52 -> 0.54 for
//     260 KB); wider planes keep one wide walker per CU.
//   * A plane's workgroup reads its own sequence first and issues its first
//     tile's loads before reducing the batch-wide state (M, validity): the
//     source range does not depend on M.
//   * The first B workgroups write the position-id and mask rows, the next
//     one the scalar outputs; they finish early and never wait.  Outputs
//     never alias inputs, so no workgroup waits for another.
#include "common.h"

namespace specv {
namespace {

// Walker shapes: lanes, 16-byte vectors per lane per tile, LDS words reserved
// (limiting residency, holding no data).
struct WalkWide {                        // 112 KB tiles; 96 KB of the CU's 160 KB LDS: one per CU
  static constexpr int kThreads = 1024, kTileVec = 7, kReserveWords = 24 * 1024;
};
struct WalkMid {                         // 56 KB tiles; 72 KB of LDS: two per CU
  static constexpr int kThreads = 512, kTileVec = 7, kReserveWords = 18 * 1024;
};
struct WalkNarrow {                      // 16 KB tiles; several per CU
  static constexpr int kThreads = 256, kTileVec = 4, kReserveWords = 0;
};

struct RealignParams {
  unsigned char *kv;
  int L, B, H, C, D, k, elt;
  int slots;                   // forward slots written per sequence: k + 1 (target) or k (draft)
  int R;                       // bytes per column (D * elt)
  long long plane_bytes;       // C * R
  int num_planes;              // L * 2 * B * H
  const int32_t *end_col, *kv_len_in, *emit_count;
  int32_t *end_col_out, *kv_len_out, *pos_ids, *mask;
  int64_t *bytes_moved;
  int32_t *status;
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Forward slots sequence b keeps: its e_b emitted tokens' worth, at most the
// slots the forward wrote.
__device__ inline int kept_slots(const RealignParams &P, int b) { return min(P.emit_count[b], P.slots); }

template <int VB>
struct VecOf;
template <>
struct VecOf<16> { using T = uint4; };
template <>
struct VecOf<8> { using T = uint2; };
template <>
struct VecOf<4> { using T = uint32_t; };
template <>
struct VecOf<2> { using T = uint16_t; };

// Makes the compiler hold a loaded value in registers at this point, so the
// load has completed (s_waitcnt) before whatever follows.
__device__ inline void hold(uint4 v) { asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w)); }
__device__ inline void hold(uint2 v) { asm volatile("" ::"v"(v.x), "v"(v.y)); }
__device__ inline void hold(uint32_t v) { asm volatile("" ::"v"(v)); }
__device__ inline void hold(uint16_t v) { asm volatile("" ::"v"(static_cast<uint32_t>(v))); }

// Streaming (non-temporal) access: every moved byte is read once and written once.
template <typename VT>
__device__ inline VT stream_ld(const VT *p) { return __builtin_nontemporal_load(p); }
__device__ inline uint4 stream_ld(const uint4 *p) {
  const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ inline uint2 stream_ld(const uint2 *p) {
  const v2u x = __builtin_nontemporal_load(reinterpret_cast<const v2u *>(p));
  return make_uint2(x.x, x.y);
}
template <typename VT>
__device__ inline void stream_st(VT v, VT *p) { __builtin_nontemporal_store(v, p); }
__device__ inline void stream_st(uint4 v, uint4 *p) {
  v4u x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<v4u *>(p));
}
__device__ inline void stream_st(uint2 v, uint2 *p) {
  v2u x = {v.x, v.y};
  __builtin_nontemporal_store(x, reinterpret_cast<v2u *>(p));
}

// Shared by every workgroup: E, M = max e_b and whether the state is valid.
// Every workgroup computes the same values from the same inputs.
template <class W>
__device__ inline void commit_state(const RealignParams &P, int *sh, int &E, int &M, bool &ok) {
  constexpr int kWaves = W::kThreads / kWave;
  E = P.end_col[0];
  int bad = (E < 0 || E > P.C - P.slots) ? 1 : 0;
  int m = 0;
  for (int b = threadIdx.x; b < P.B; b += blockDim.x) {
    const int n = P.kv_len_in[b], e = P.emit_count[b];
    if (n < 0 || n > E || e < 0 || e > P.k + 1) bad = 1;
    m = max(m, min(e, P.slots));
  }
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int wb = wave_max_i(bad), wmx = wave_max_i(m);
  if (lane == 0) {
    sh[w] = wb;
    sh[kWaves + w] = wmx;
  }
  __syncthreads();
  int allbad = 0, mm = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    allbad = max(allbad, sh[i]);
    mm = max(mm, sh[kWaves + i]);
  }
  __syncthreads();
  ok = allbad == 0;
  M = mm;
}

// Address of vector i of a plane.  With 32-bit indices (planes under 2 GiB)
// the byte offset is a 32-bit lane value added to the plane's base, which
// sits in scalar registers: one VGPR per address instead of two, which leaves
// room for wider tiles.
template <typename VT, typename IT>
__device__ inline VT *cell(unsigned char *pb, IT i) {
  if constexpr (sizeof(IT) == 4)
    return reinterpret_cast<VT *>(pb + static_cast<uint32_t>(i) * static_cast<uint32_t>(sizeof(VT)));
  else
    return reinterpret_cast<VT *>(pb + static_cast<size_t>(i) * sizeof(VT));
}

// One plane: the moved range [E - n, E + e) shifted right by M - e columns,
// walked from right to left in tiles.  The plane's own sequence is read first
// and, when it can move, the first tile's loads are issued before the
// batch-wide state (M, validity) is reduced: the source range does not depend
// on M.  Loads are checked against this sequence's own values, so they stay in
// bounds whatever the rest of the batch holds; nothing is stored unless the
// whole batch is valid.  IT indexes vectors within the plane: int when the
// plane is under 2 GiB, long long otherwise.
template <class W, int VB, typename IT>
__device__ inline void move_plane(const RealignParams &P, int p, int b, int *sh) {
  using VT = typename VecOf<VB>::T;
  constexpr int kThreads = W::kThreads, kTileVec = W::kTileVec;
  const int E0 = P.end_col[0];
  const int n = P.kv_len_in[b], e_in = P.emit_count[b];
  const int e = min(e_in, P.slots);
  // e == slots: this sequence kept the most any can, so it does not move
  const bool may_move = E0 >= 0 && E0 <= P.C - P.slots && n >= 0 && n <= E0 && e_in >= 0 &&
                        e_in <= P.k + 1 && e < P.slots && n + e > 0;
  const IT per_col = P.R / VB;                              // vectors per column
  unsigned char *pb = P.kv + static_cast<size_t>(p) * P.plane_bytes;
  const IT lo = static_cast<IT>(E0 - n) * per_col;          // first source vector
  constexpr int TV = kThreads * kTileVec;                    // vectors per tile
  const int t = threadIdx.x;
  IT hi = lo + static_cast<IT>(n + e) * per_col;             // one past the last source vector

  // Every lane issues every load and store of a tile (no per-lane branches),
  // so the compiler counts the memory operations in flight exactly and the
  // wait for a tile's loads leaves the next tile's loads and the previous
  // tile's stores in flight (a branch per access makes it wait for all of
  // them).  Lanes left of the moved range (only in its leftmost tile) load
  // its first cell and store that value back to the same cell: that cell is
  // never a destination of the right shift, so the store changes nothing.
  // Three register buffers rotate: no copy between them (a copy would wait
  // for the next tile's loads), and a buffer is reloaded two steps after its
  // stores were issued (reloading it right away waits for those stores).
  VT buf0[kTileVec], buf1[kTileVec], buf2[kTileVec];
  if (may_move) {
#pragma unroll
    for (int u = 0; u < kTileVec; ++u) buf0[u] = stream_ld(cell<VT>(pb, max(hi - TV + u * kThreads + t, lo)));
  }
  int E, M;
  bool ok;
  commit_state<W>(P, sh, E, M, ok);        // barriers: every lane of the workgroup gets here
  if (!ok || !may_move || M == e) return;  // uniform in the workgroup
  const IT shift = static_cast<IT>(M - e) * per_col;
  // One step: load the tile left of `hi` (after the last tile: the first
  // cell again, unused), wait for the current tile's loads in every lane,
  // store it `shift` to the right.  Returns whether a tile is left.
  auto step = [&](VT (&cur)[kTileVec], VT (&nxt)[kTileVec]) {
    const IT nhi = hi - TV;
#pragma unroll
    for (int u = 0; u < kTileVec; ++u) nxt[u] = stream_ld(cell<VT>(pb, max(nhi - TV + u * kThreads + t, lo)));
#pragma unroll
    for (int u = 0; u < kTileVec; ++u) hold(cur[u]);          // this tile's loads have landed
    __syncthreads();                                           // ... in every lane
#pragma unroll
    for (int u = 0; u < kTileVec; ++u) {
      const IT i = hi - TV + u * kThreads + t;
      stream_st(cur[u], cell<VT>(pb, i >= lo ? i + shift : lo));
    }
    hi = nhi;
    return nhi > lo;                        // uniform
  };
  while (step(buf0, buf1) && step(buf1, buf2) && step(buf2, buf0)) {
  }
}

template <class W, int VB, typename IT>
__global__ __launch_bounds__(W::kThreads) void realign_kernel(RealignParams P) {
  constexpr int kThreads = W::kThreads, kWaves = kThreads / kWave;
  __shared__ int sh[2 * kWaves];
  __shared__ long long sh_bytes[kWaves];
  if constexpr (W::kReserveWords > 0) {
    __shared__ uint32_t sh_reserve[W::kReserveWords];
    asm volatile("" ::"s"(sh_reserve));    // keep the reservation (it limits residency, holds no data)
  }
  const int blk = blockIdx.x;
  const int t = threadIdx.x;
  if (blk > P.B) {                         // one plane, address order: p = ((l * 2 + kv) * B + b) * H + h
    const int p = blk - P.B - 1;
    move_plane<W, VB, IT>(P, p, (p / P.H) % P.B, sh);
    return;
  }
  int E, M;
  bool ok;
  commit_state<W>(P, sh, E, M, ok);

  if (blk < P.B) {                         // position ids and mask of one sequence
    if (!ok) return;
    const int b = blk;
    const int En = E + M;
    const int start = En - (P.kv_len_in[b] + kept_slots(P, b));
    int32_t *pos = P.pos_ids ? P.pos_ids + static_cast<size_t>(b) * P.C : nullptr;
    int32_t *msk = P.mask ? P.mask + static_cast<size_t>(b) * P.C : nullptr;
    for (int c = t; c < P.C; c += kThreads) {
      const bool in = c >= start && c < En;
      if (msk) msk[c] = in ? 1 : 0;
      if (pos) pos[c] = in ? c - start : 0;
    }
    return;
  }
  // scalar outputs
  if (!ok) {
    if (P.status) {
      const bool cap = E < 0 || E > P.C - P.slots;
      for (int b = t; b < P.B; b += kThreads) {
        const int n = P.kv_len_in[b], e = P.emit_count[b];
        int st = cap ? SPEC_ST_CAPACITY : 0;
        if (n < 0 || n > E || e < 0 || e > P.k + 1) st |= SPEC_ST_BAD_STATE;
        P.status[b] = st;
      }
    }
    return;
  }
  long long moved = 0;
  for (int b = t; b < P.B; b += kThreads) {
    const int e = kept_slots(P, b);
    const int n1 = P.kv_len_in[b] + e;
    P.kv_len_out[b] = n1;
    if (P.status) P.status[b] = 0;
    if (e != M) moved += n1;
  }
  const int lane = t & (kWave - 1), w = t / kWave;
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) moved += __shfl_xor(moved, m, kWave);
  if (lane == 0) sh_bytes[w] = moved;
  __syncthreads();
  if (t == 0) {
    long long tot = 0;
    for (int i = 0; i < kWaves; ++i) tot += sh_bytes[i];
    *P.end_col_out = E + M;
    if (P.bytes_moved) *P.bytes_moved = 2LL * tot * P.L * 2LL * P.H * P.R;
  }
}

// ---- tree verification: move the accepted path's slots together -----------
// The forward over a candidate tree wrote one slot per node at columns E + i.
// Sequence b keeps the slots path[b, 0..e_b-1] (increasing node indices, path
// starting at the root 0) and they must sit at columns E .. E + e_b - 1 before
// the usual realignment.  A valid path has path[j] >= j, with equality
// exactly on a prefix j < j0 (once a node is skipped every later one sits
// further right), so the slots to move are the contiguous tail j0 .. e_b - 1.
// Column j receives column path[j] > j: it is never the source of a later j'
// (path[j'] > path[j]) but may be the source of an earlier one, so every pass
// reads all of its sources before any of its writes (registers, then a
// barrier), and each plane's units go in increasing j across passes.
//
// One workgroup per (sequence, layer, K/V, group of heads): the group's
// planes lie hpb * C * R bytes apart at most, and the workgroup reads the
// sequence's path once, checking it in parallel, instead of once per plane.
constexpr int kCompactThreads = 256;
constexpr int kCompactU = 4;
static_assert(kCompactThreads >= SPEC_TREE_MAX_N, "one lane per tree node");

struct CompactParams {
  unsigned char *kv;
  int B, H, C, N, R;           // R: bytes per column
  int hpb, hsplit;             // heads per workgroup, workgroups per (layer, K/V, sequence)
  long long plane_bytes;
  const int32_t *end_col, *path, *emit_count;
  int32_t *status;
};

template <int VB>
__global__ __launch_bounds__(kCompactThreads) void tree_compact_kernel(CompactParams P) {
  using VT = typename VecOf<VB>::T;
  const int t = threadIdx.x;
  const int blk = blockIdx.x;
  const int b = blk % P.B;                  // consecutive workgroups: consecutive sequences
  const int rest = blk / P.B;
  const int hs = rest % P.hsplit;
  const int lk = rest / P.hsplit;           // layer * 2 + (K or V)
  // the path row is read with the counts (one round of loads): lanes t < N
  // read entries t and t - 1, used where t < e
  const int32_t *pb = P.path + static_cast<size_t>(b) * P.N;
  int node_t = -1, prev_t = -1;
  if (t < P.N) {
    node_t = pb[t];
    if (t > 0) prev_t = pb[t - 1];
  }
  const int E = P.end_col[0];
  const int e = P.emit_count[b];
  const bool shape_ok = E >= 0 && E <= P.C - P.N && e >= 0 && e <= P.N;
  int node = -1, prev = -1;
  if (shape_ok && t < e) {
    node = node_t;
    prev = prev_t;
  }
  const bool lane_ok = t >= e || (node > prev && node < P.N && (t > 0 || node == 0));
  const bool ok = shape_ok && __syncthreads_and(lane_ok);
  if (P.status && lk == 0 && hs == 0 && t == 0) P.status[b] = ok ? 0 : SPEC_ST_BAD_STATE;
  if (!ok) return;
  __shared__ int sh_path[SPEC_TREE_MAX_N];
  if (t < e) sh_path[t] = node;
  const int j0 = __syncthreads_count(t < e && node == t);   // barrier: sh_path is visible
  const int moved = e - j0;
  const int h0 = hs * P.hpb;
  const int nh = min(P.hpb, P.H - h0);
  if (moved <= 0 || nh <= 0) return;
  const int per_col = P.R / VB;
  const int per_plane = moved * per_col;     // (column j0 + m, vector v) pairs, column-major
  const int units = nh * per_plane;
  const size_t plane0 = (static_cast<size_t>(lk) * P.B + b) * P.H + h0;
  unsigned char *base = P.kv + plane0 * P.plane_bytes;
  constexpr int kPass = kCompactThreads * kCompactU;
  for (int u0 = 0; u0 < units; u0 += kPass) {
    VT x[kCompactU];
    VT *dst[kCompactU];
#pragma unroll
    for (int q = 0; q < kCompactU; ++q) {
      const int u = u0 + q * kCompactThreads + t;
      dst[q] = nullptr;
      if (u < units) {
        const int h = u / per_plane;
        const int r = u - h * per_plane;
        const int m = r / per_col;
        const int v = r - m * per_col;
        const int j = j0 + m;
        VT *pl = reinterpret_cast<VT *>(base + static_cast<size_t>(h) * P.plane_bytes);
        x[q] = pl[static_cast<size_t>(E + sh_path[j]) * per_col + v];
        dst[q] = pl + static_cast<size_t>(E + j) * per_col + v;
      }
    }
#pragma unroll
    for (int q = 0; q < kCompactU; ++q)
      if (dst[q]) hold(x[q]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCompactU; ++q)
      if (dst[q]) *dst[q] = x[q];
    __syncthreads();
  }
}

}  // namespace
}  // namespace specv

using namespace specv;

template <class W, typename IT>
static void launch_realign(const RealignParams &P, size_t R, const void *kv, dim3 grid, hipStream_t s) {
  const dim3 block(W::kThreads);
  if (R % 16 == 0 && aligned(kv, 16))
    hipLaunchKernelGGL((realign_kernel<W, 16, IT>), grid, block, 0, s, P);
  else if (R % 8 == 0 && aligned(kv, 8))
    hipLaunchKernelGGL((realign_kernel<W, 8, IT>), grid, block, 0, s, P);
  else if (R % 4 == 0 && aligned(kv, 4))
    hipLaunchKernelGGL((realign_kernel<W, 4, IT>), grid, block, 0, s, P);
  else
    hipLaunchKernelGGL((realign_kernel<W, 2, IT>), grid, block, 0, s, P);
}

static int realign_launch(void *kv, spec_dtype dt, int L, int B, int H, int C, int D, int k, int slots,
                          const int32_t *end_col, const int32_t *kv_len_in, const int32_t *emit_count,
                          int32_t *end_col_out, int32_t *kv_len_out, int32_t *pos_ids, int32_t *mask,
                          int64_t *bytes_moved, int32_t *status, spec_stream_t stream) {
  if (!kv || !end_col || !kv_len_in || !emit_count || !end_col_out || !kv_len_out) return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (L < 1 || B < 1 || H < 1 || C < 1 || D < 1 || k < 1) return SPEC_EINVAL;
  const int elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(kv, elt)) return SPEC_EINVAL;
  const long long planes = 2LL * L * B * H;
  const long long R = static_cast<long long>(D) * elt;
  if (planes + B + 1 >= INT32_MAX || R >= INT32_MAX || static_cast<long long>(C) * R >= (1LL << 62) / planes)
    return SPEC_EINVAL;
  const size_t kv_bytes = static_cast<size_t>(planes) * C * R;
  const size_t bc = static_cast<size_t>(B) * C * 4;
  const void *ins[] = {kv, end_col, kv_len_in, emit_count};
  const size_t in_n[] = {kv_bytes, 4, static_cast<size_t>(B) * 4, static_cast<size_t>(B) * 4};
  const void *outs[] = {end_col_out, kv_len_out, pos_ids, mask, bytes_moved, status};
  const size_t out_n[] = {4, static_cast<size_t>(B) * 4, bc, bc, 8, static_cast<size_t>(B) * 4};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }

  RealignParams P;
  P.kv = static_cast<unsigned char *>(kv);
  P.L = L;
  P.B = B;
  P.H = H;
  P.C = C;
  P.D = D;
  P.k = k;
  P.slots = slots;
  P.elt = elt;
  P.R = static_cast<int>(R);
  P.plane_bytes = static_cast<long long>(C) * R;
  P.num_planes = static_cast<int>(planes);
  P.end_col = end_col;
  P.kv_len_in = kv_len_in;
  P.emit_count = emit_count;
  P.end_col_out = end_col_out;
  P.kv_len_out = kv_len_out;
  P.pos_ids = pos_ids;
  P.mask = mask;
  P.bytes_moved = bytes_moved;
  P.status = status;
  const dim3 grid(static_cast<unsigned>(B + 1 + planes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  constexpr long long kWideTileBytes = 16LL * WalkWide::kThreads * WalkWide::kTileVec;
  constexpr long long kMidPlaneBytes = 512LL << 10;
  if (P.plane_bytes < kWideTileBytes)      // a plane smaller than one wide tile: narrow walkers
    launch_realign<WalkNarrow, int>(P, R, kv, grid, s);
  else if (P.plane_bytes < kMidPlaneBytes) // planes of a few wide tiles: two walkers per CU
    launch_realign<WalkMid, int>(P, R, kv, grid, s);
  else if (P.plane_bytes < (1LL << 31))    // vector indices and byte offsets fit 32 bits
    launch_realign<WalkWide, int>(P, R, kv, grid, s);
  else
    launch_realign<WalkWide, long long>(P, R, kv, grid, s);
  return launch_status();
}

extern "C" int spec_commit_realign_kv(void *kv, spec_dtype dt, int L, int B, int H, int C, int D, int k,
                                      const int32_t *end_col, const int32_t *kv_len_in,
                                      const int32_t *emit_count, int32_t *end_col_out,
                                      int32_t *kv_len_out, int32_t *pos_ids, int32_t *mask,
                                      int64_t *bytes_moved, int32_t *status, spec_stream_t stream) {
  if (!pos_ids || !mask) return SPEC_EINVAL;
  return realign_launch(kv, dt, L, B, H, C, D, k, k + 1, end_col, kv_len_in, emit_count, end_col_out,
                        kv_len_out, pos_ids, mask, bytes_moved, status, stream);
}

extern "C" int spec_resync_draft_kv(void *kv, spec_dtype dt, int L, int B, int H, int C, int D, int k,
                                    const int32_t *end_col, const int32_t *kv_len_in,
                                    const int32_t *emit_count, int32_t *end_col_out,
                                    int32_t *kv_len_out, int32_t *pos_ids, int32_t *mask,
                                    int64_t *bytes_moved, int32_t *status, spec_stream_t stream) {
  return realign_launch(kv, dt, L, B, H, C, D, k, k, end_col, kv_len_in, emit_count, end_col_out,
                        kv_len_out, pos_ids, mask, bytes_moved, status, stream);
}

extern "C" int spec_compact_tree_kv(void *kv, spec_dtype dt, int L, int B, int H, int C, int D, int N,
                                    const int32_t *end_col, const int32_t *path,
                                    const int32_t *emit_count, int32_t *status, spec_stream_t stream) {
  if (!kv || !end_col || !path || !emit_count) return SPEC_EINVAL;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_EINVAL;
  if (L < 1 || B < 1 || H < 1 || C < 1 || D < 1 || N < 1) return SPEC_EINVAL;
  if (N > SPEC_TREE_MAX_N) return SPEC_ECAPACITY;
  const int elt = dt == SPEC_BF16 ? 2 : 4;
  if (!aligned(kv, elt)) return SPEC_EINVAL;
  const long long planes = 2LL * L * B * H;
  const long long R = static_cast<long long>(D) * elt;
  if (planes + B >= INT32_MAX || static_cast<long long>(C) * R / elt >= INT32_MAX ||
      static_cast<long long>(C) * R >= (1LL << 62) / planes || static_cast<long long>(H) * N * R >= INT32_MAX)
    return SPEC_EINVAL;
  const size_t kv_bytes = static_cast<size_t>(planes) * C * R;
  const size_t b4 = static_cast<size_t>(B) * 4;
  if (overlaps(status, b4, kv, kv_bytes) || overlaps(status, b4, path, b4 * N) ||
      overlaps(status, b4, emit_count, b4) || overlaps(status, b4, end_col, 4))
    return SPEC_EINVAL;
  // enough workgroups to fill the chip: split each sequence's heads when the
  // (sequence, layer, K/V) count alone is small
  const long long groups = static_cast<long long>(B) * 2 * L;
  const int hsplit = static_cast<int>(std::min<long long>(H, std::max<long long>(1, (2048 + groups - 1) / groups)));
  const int hpb = (H + hsplit - 1) / hsplit;
  CompactParams P;
  P.kv = static_cast<unsigned char *>(kv);
  P.B = B;
  P.H = H;
  P.C = C;
  P.N = N;
  P.R = static_cast<int>(R);
  P.hpb = hpb;
  P.hsplit = (H + hpb - 1) / hpb;
  P.plane_bytes = static_cast<long long>(C) * R;
  P.end_col = end_col;
  P.path = path;
  P.emit_count = emit_count;
  P.status = status;
  const dim3 grid(static_cast<unsigned>(groups * P.hsplit)), block(kCompactThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (R % 16 == 0 && aligned(kv, 16))
    hipLaunchKernelGGL(tree_compact_kernel<16>, grid, block, 0, s, P);
  else if (R % 8 == 0 && aligned(kv, 8))
    hipLaunchKernelGGL(tree_compact_kernel<8>, grid, block, 0, s, P);
  else if (R % 4 == 0 && aligned(kv, 4))
    hipLaunchKernelGGL(tree_compact_kernel<4>, grid, block, 0, s, P);
  else
    hipLaunchKernelGGL(tree_compact_kernel<2>, grid, block, 0, s, P);
  return launch_status();
}
