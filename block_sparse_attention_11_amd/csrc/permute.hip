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

// V in Hilbert order as one transposed [d][block] tile per key block:
//   tile row c holds column c of the block's rows (padding keys are 0), in
//   8-byte units of 4 keys; inside each 16-key group the units are stored in
//   the order 0, 2, 1, 3 (vt_pos), so the 8 keys one lane of the attention
//   kernel's P.V MFMA needs are one 16-byte read.
// A thread moves a 4-key x 8-column unit: four 16-byte row loads, eight 8-byte
// stores (byte shuffles with v_perm_b32); lanes run key-group fastest so 32
// lanes write 256 contiguous bytes of one tile row.
__global__ __launch_bounds__(kPermuteThreads) void pack_v_kernel(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
    const int32_t* __restrict__ index, int n, int d, int block, int nb) {
  const int h = blockIdx.z;
  const int j = blockIdx.y;
  const int kgroups = block / 4;
  const int units = kgroups * (d / 8);
  const int g = blockIdx.x * kPermuteThreads + threadIdx.x;
  if (g >= units) return;
  const int kq = g % kgroups;
  const int c8 = g / kgroups;
  const uint16_t* sh = src + (size_t)h * n * d;
  uint4 rows[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int r = j * block + 4 * kq + x;
    rows[x] = make_uint4(0u, 0u, 0u, 0u);
    if (r < n) rows[x] = *reinterpret_cast<const uint4*>(sh + (size_t)index[r] * d + 8 * c8);
  }
  uint16_t* tile = dst + (((size_t)h * nb + j) * d) * block;
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const uint32_t w0 = dd < 2 ? rows[0].x : dd < 4 ? rows[0].y : dd < 6 ? rows[0].z : rows[0].w;
    const uint32_t w1 = dd < 2 ? rows[1].x : dd < 4 ? rows[1].y : dd < 6 ? rows[1].z : rows[1].w;
    const uint32_t w2 = dd < 2 ? rows[2].x : dd < 4 ? rows[2].y : dd < 6 ? rows[2].z : rows[2].w;
    const uint32_t w3 = dd < 2 ? rows[3].x : dd < 4 ? rows[3].y : dd < 6 ? rows[3].z : rows[3].w;
    const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
    uint2 o;
    o.x = __builtin_amdgcn_perm(w1, w0, sel);
    o.y = __builtin_amdgcn_perm(w3, w2, sel);
    const int row = 8 * c8 + dd;
    *reinterpret_cast<uint2*>(tile + (size_t)row * block + vt_pos(4 * kq)) = o;
  }
}

}  // namespace

hipError_t launch_pack_v(const void* src, void* dst, const int32_t* index, int heads,
                         int n, int d, int block, hipStream_t s) {
  const int nb = (n + block - 1) / block;
  const int units = (block / 4) * (d / 8);
  hipLaunchKernelGGL(pack_v_kernel, dim3((units + kPermuteThreads - 1) / kPermuteThreads, nb, heads),
                     dim3(kPermuteThreads), 0, s, (const uint16_t*)src, (uint16_t*)dst,
                     index, n, d, block, nb);
  return hipGetLastError();
}

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
