// Row gather dst[h][r][:] = src[h][index[r]][:]: puts Q/K/V into Hilbert
// order and O back into token order (aixai.ru FVAttn post, "Sparse-routing
// frontend": blocks are formed along the curve).
//
// HBM-bound copy.  Each lane moves one 16-byte vector; the rows of a head are
// laid out along blockIdx.x and heads along blockIdx.y, so the source row is
// found with one index load per row and no 64-bit division.
#include "internal.h"

namespace fvattn {
namespace {

constexpr int kPermuteThreads = 256;
constexpr int kPermuteVecPerThread = 4;

template <typename V>
__global__ __launch_bounds__(kPermuteThreads) void permute_rows_kernel(
    const V* __restrict__ src, V* __restrict__ dst,
    const int32_t* __restrict__ index, int n, uint32_t vec_per_row) {
  const size_t head_vecs = (size_t)n * vec_per_row;
  const V* s = src + (size_t)blockIdx.y * head_vecs;
  V* d = dst + (size_t)blockIdx.y * head_vecs;
  const uint32_t base =
      (uint32_t)blockIdx.x * (kPermuteThreads * kPermuteVecPerThread) + threadIdx.x;
  V tmp[kPermuteVecPerThread];
  uint32_t g[kPermuteVecPerThread];
#pragma unroll
  for (int e = 0; e < kPermuteVecPerThread; ++e) {
    g[e] = base + e * kPermuteThreads;
    if (g[e] < head_vecs) {
      const uint32_t r = g[e] / vec_per_row;
      const uint32_t c = g[e] - r * vec_per_row;
      tmp[e] = s[(size_t)index[r] * vec_per_row + c];
    }
  }
#pragma unroll
  for (int e = 0; e < kPermuteVecPerThread; ++e)
    if (g[e] < head_vecs) d[g[e]] = tmp[e];
}

template <typename V>
hipError_t launch_typed(const void* src, void* dst, const int32_t* index,
                        int heads, int n, size_t row_bytes, hipStream_t s) {
  const uint32_t vpr = (uint32_t)(row_bytes / sizeof(V));
  const size_t head_vecs = (size_t)n * vpr;
  const size_t per_block = (size_t)kPermuteThreads * kPermuteVecPerThread;
  const unsigned gx = (unsigned)((head_vecs + per_block - 1) / per_block);
  hipLaunchKernelGGL(permute_rows_kernel<V>, dim3(gx, heads),
                     dim3(kPermuteThreads), 0, s, (const V*)src, (V*)dst, index,
                     n, vpr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_rows(const void* src, void* dst, const int32_t* index,
                               int heads, int n, size_t row_bytes,
                               hipStream_t s) {
  const uintptr_t align = (uintptr_t)src | (uintptr_t)dst;
  if (row_bytes % 16 == 0 && align % 16 == 0)
    return launch_typed<uint4>(src, dst, index, heads, n, row_bytes, s);
  if (row_bytes % 4 == 0 && align % 4 == 0)
    return launch_typed<uint32_t>(src, dst, index, heads, n, row_bytes, s);
  return launch_typed<uint16_t>(src, dst, index, heads, n, row_bytes, s);
}

}  // namespace fvattn
