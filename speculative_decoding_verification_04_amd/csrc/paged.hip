// Commit for a variable-length (paged) KV layout: rollback only (gfx950).
//
// The "Correctness Forensics for Batch Speculative Decoding" summary (section 2
// and App. F) notes that variable-length layouts need no repadding, but the
// rejected tokens must still be rolled back in the position ids and the KV
// cache.  With a paged cache the rollback moves no KV bytes: sequence b keeps
// n'_b = n_b + e_b rows (the last emitted token has no KV yet: App. D), its
// next input position is n'_b, and the block-table pages that the verify
// forward's k + 1 slots needed beyond ceil(n'_b / page) are released.
//
// Design.  One 1024-lane workgroup walks the batch a tile of sequences at a
// time: one lane per sequence computes its lengths and its count of released
// pages, a block prefix sum (with a carry across tiles) gives each sequence's
// offset into the released list, and every lane then copies its released
// block-table entries in order.  The work is a few integers per sequence;
// the call is launch-latency bound.
#include "common.h"

namespace specv {
namespace {

constexpr int kPagedThreads = 1024;

struct PagedParams {
  int B, k, page, max_pages;
  const int32_t *kv_len_in, *emit_count, *block_table;
  int32_t *kv_len_out, *pages_kept, *freed, *freed_offsets, *status;
};

__device__ inline long long pages_for(long long rows, int page) { return (rows + page - 1) / page; }

__global__ __launch_bounds__(kPagedThreads) void paged_commit_kernel(PagedParams P) {
  __shared__ int sh_scan[kPagedThreads / kWave + 1];
  const int t = threadIdx.x;
  int carry = 0;
  for (int b0 = 0; b0 < P.B; b0 += kPagedThreads) {
    const int b = b0 + t;
    int cnt = 0, keep = 0;
    if (b < P.B) {
      const long long n = P.kv_len_in[b];
      const int e = P.emit_count[b];
      int st = 0;
      if (n < 0 || e < 0 || e > P.k + 1) st |= SPEC_ST_BAD_STATE;
      else if (pages_for(n + P.k + 1, P.page) > P.max_pages) st |= SPEC_ST_CAPACITY;
      if (st) {
        P.kv_len_out[b] = static_cast<int32_t>(n);
        keep = n > 0 ? static_cast<int>(pages_for(n, P.page)) : 0;
      } else {
        const long long used = pages_for(n + P.k + 1, P.page);
        keep = static_cast<int>(pages_for(n + e, P.page));
        cnt = static_cast<int>(used - keep);
        P.kv_len_out[b] = static_cast<int32_t>(n + e);
      }
      P.pages_kept[b] = keep;
      if (P.status) P.status[b] = st;
    }
    int total;
    const int ex = block_excl_scan(cnt, sh_scan, &total);
    if (b < P.B) {
      const int off = carry + ex;
      P.freed_offsets[b] = off;
      const int32_t *row = P.block_table + static_cast<size_t>(b) * P.max_pages;
      for (int i = 0; i < cnt; ++i) P.freed[off + i] = row[keep + i];
    }
    carry += total;
  }
  if (t == 0) P.freed_offsets[P.B] = carry;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" int spec_commit_paged(int B, int k, int page_size, int max_pages, const int32_t *kv_len_in,
                                 const int32_t *emit_count, const int32_t *block_table,
                                 int32_t *kv_len_out, int32_t *pages_kept, int32_t *freed_pages,
                                 int32_t *freed_offsets, int32_t *status, spec_stream_t stream) {
  if (!kv_len_in || !emit_count || !block_table || !kv_len_out || !pages_kept || !freed_pages ||
      !freed_offsets)
    return SPEC_EINVAL;
  if (B < 1 || k < 1 || page_size < 1 || max_pages < 1) return SPEC_EINVAL;
  if (static_cast<long long>(B) * max_pages >= INT32_MAX) return SPEC_EINVAL;
  const long long per = (static_cast<long long>(k) + page_size) / page_size;   // ceil((k+1)/page)
  if (B * per >= INT32_MAX) return SPEC_EINVAL;
  const size_t b4 = static_cast<size_t>(B) * 4;
  const void *ins[] = {kv_len_in, emit_count, block_table};
  const size_t in_n[] = {b4, b4, static_cast<size_t>(B) * max_pages * 4};
  void *outs[] = {kv_len_out, pages_kept, freed_pages, freed_offsets, status};
  const size_t out_n[] = {b4, b4, static_cast<size_t>(B * per) * 4, b4 + 4, b4};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return SPEC_EINVAL;
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return SPEC_EINVAL;
  }
  PagedParams P;
  P.B = B;
  P.k = k;
  P.page = page_size;
  P.max_pages = max_pages;
  P.kv_len_in = kv_len_in;
  P.emit_count = emit_count;
  P.block_table = block_table;
  P.kv_len_out = kv_len_out;
  P.pages_kept = pages_kept;
  P.freed = freed_pages;
  P.freed_offsets = freed_offsets;
  P.status = status;
  (void)hipGetLastError();
  hipLaunchKernelGGL(paged_commit_kernel, dim3(1), dim3(kPagedThreads), 0, static_cast<hipStream_t>(stream), P);
  return launch_status();
}
