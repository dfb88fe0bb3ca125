// Read floor for the greedy verification's streaming pass (bench.py only; not
// part of the library).  The same row-aligned chunks of 16384 bf16 logits as
// the verification's producers, 512 lanes per workgroup with four 16-byte
// non-temporal loads in flight per lane, each chunk reduced to its maximum and
// stored: one pass over the logits with no argmax, no publication and no
// commit.  Its time per launch over the verification's own buffers is what
// any single pass over those bytes costs on this GPU.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kU = 4;
constexpr int kVec = 8;                         // bf16 per 16-byte vector
constexpr int kChunk = kThreads * kU * kVec;    // 16384 logits

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ inline float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(kThreads) void floor_max_kernel(const uint16_t *logits, int V, int chunks, float *out) {
  __shared__ float sh[kThreads / 64];
  const int blk = blockIdx.x, row = blk / chunks, c = blk - row * chunks;
  const uint16_t *rowp = logits + static_cast<size_t>(row) * V;
  const int s = c * kChunk, e = min(V, s + kChunk);
  const int nv = (e - s) / kVec;                 // whole vectors (rows start 16-byte aligned)
  // every load is issued before any is used (four in flight per lane)
  v4u x[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int vi = threadIdx.x + u * kThreads;
    x[u] = vi < nv ? __builtin_nontemporal_load(reinterpret_cast<const v4u *>(rowp + s + vi * kVec))
                   : v4u{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};   // bf16 -inf
  }
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < kU; ++u)
    m = fmaxf(m, fmaxf(fmaxf(fmaxf(lo16(x[u].x), hi16(x[u].x)), fmaxf(lo16(x[u].y), hi16(x[u].y))),
                       fmaxf(fmaxf(lo16(x[u].z), hi16(x[u].z)), fmaxf(lo16(x[u].w), hi16(x[u].w)))));
  for (int v = s + nv * kVec + threadIdx.x; v < e; v += kThreads) m = fmaxf(m, __uint_as_float(static_cast<uint32_t>(rowp[v]) << 16));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = sh[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, sh[i]);
    out[blk] = r;
  }
}

}  // namespace

// Chunk maxima of rows [rows, V] of bf16 logits (16-byte aligned rows: V a
// multiple of 8 and an aligned base); out holds rows * ceil(V / 16384) floats.
// Returns the number of chunks, or -1 for bad arguments.
extern "C" int floor_chunk_max_bf16(const void *logits, int rows, int V, float *out, void *stream) {
  if (!logits || !out || rows < 1 || V < 1 || V % kVec != 0 || (reinterpret_cast<uintptr_t>(logits) & 15u)) return -1;
  const int chunks = (V + kChunk - 1) / kChunk;
  const long long n = static_cast<long long>(rows) * chunks;
  if (n >= INT32_MAX) return -1;
  hipLaunchKernelGGL(floor_max_kernel, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(logits), V, chunks, out);
  return hipGetLastError() == hipSuccess ? static_cast<int>(n) : -1;
}
