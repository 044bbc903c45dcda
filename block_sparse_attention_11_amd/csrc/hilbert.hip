// Hilbert order of the (t, y, x) token grid.
//
// The routing frontend regroups tokens along a Hilbert curve so that nearby
// tokens share or neighbour blocks (aixai.ru FVAttn post, "Sparse-routing
// frontend").  Curve: J. Skilling's 3D construction ("Programming the Hilbert
// curve", AIP Conf. Proc. 707, 2004) on the enclosing cube of side 2^b, axis
// order (t, y, x), index bits interleaved MSB first with t on top.
//
// GPU formulation (no sort, no workspace): walk the curve itself.  The index
// range [0, 8^b) is cut into aligned chunks of 8^m indices; by the nesting
// property of the curve each chunk covers one aligned 2^m sub-cube, and each
// coarser aligned run of 8^(m+l) indices covers an aligned 2^(m+l) cube.  A
// workgroup owns one chunk:
//   1. its output offset = number of grid points on the curve before the
//      chunk = sum, over the levels above the chunk, of the grid points inside
//      the sibling cubes that come earlier at that level (box counts, one
//      decode per sibling);
//   2. it decodes its 8^m indices to points, keeps those inside the grid and
//      writes perm / inv_perm at offset + (exclusive scan of the in-grid flags).
// The ranks equal "sort grid points by curve index", with no comparison sort.
#include "device_util.h"
#include "internal.h"

namespace fvattn {
namespace {

constexpr int kHilbertThreads = 256;
constexpr int kMaxChunkBits = 4;                 // chunk = 8^4 = 4096 indices
constexpr int kMaxPerThread = (1 << (3 * kMaxChunkBits)) / kHilbertThreads;  // 16

// Index -> point on the b-bit 3D curve.
__device__ inline void hilbert_decode(uint32_t h, int b, uint32_t& t,
                                      uint32_t& y, uint32_t& x) {
  // De-interleave: bit q of axis a is index bit 3q + (2 - a).
  uint32_t w0 = 0, w1 = 0, w2 = 0;
  for (int q = 0; q < b; ++q) {
    w0 |= ((h >> (3 * q + 2)) & 1u) << q;
    w1 |= ((h >> (3 * q + 1)) & 1u) << q;
    w2 |= ((h >> (3 * q + 0)) & 1u) << q;
  }
  // Gray decode across the three words.
  const uint32_t g = w2 >> 1;
  w2 ^= w1;
  w1 ^= w0;
  w0 ^= g;
  // Redo the excess work from the finest level up, last axis first.
  const uint32_t top = 1u << b;
  for (uint32_t Q = 2; Q != top; Q <<= 1) {
    const uint32_t low = Q - 1;
    // axis 2
    if (w2 & Q) {
      w0 ^= low;
    } else {
      const uint32_t s = (w0 ^ w2) & low;
      w0 ^= s;
      w2 ^= s;
    }
    // axis 1
    if (w1 & Q) {
      w0 ^= low;
    } else {
      const uint32_t s = (w0 ^ w1) & low;
      w0 ^= s;
      w1 ^= s;
    }
    // axis 0 against itself: the exchange is a no-op, the reflection is not
    if (w0 & Q) w0 ^= low;
  }
  t = w0;
  y = w1;
  x = w2;
}

__device__ inline int64_t clipped(uint32_t origin, uint32_t side, int dim) {
  const int64_t lo = origin;
  const int64_t hi = min<int64_t>((int64_t)origin + side, (int64_t)dim);
  return hi > lo ? hi - lo : 0;
}

__global__ __launch_bounds__(kHilbertThreads) void hilbert_chunk_kernel(
    int T, int Y, int X, int b, int m, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv) {
  const int32_t n_total = T * Y * X;
  __shared__ int64_t s_red[kHilbertThreads / kWave];
  __shared__ int32_t s_scan[kHilbertThreads / kWave];
  const uint32_t c = blockIdx.x;
  const int L = b - m;                       // levels above the chunk
  const int tid = threadIdx.x;

  // 1. points of the grid on the curve before this chunk.
  int64_t before = 0;
  if (tid < 7 * L) {
    const int lev = tid / 7 + 1;             // 1 = coarsest level
    const uint32_t sib = tid % 7;
    const uint32_t digit = (c >> (3 * (L - lev))) & 7u;
    if (sib < digit) {
      const uint32_t above = c >> (3 * (L - lev + 1));
      const uint32_t prefix = (above << 3) | sib;
      const uint32_t first = prefix << (3 * (L - lev) + 3 * m);
      uint32_t pt, py, px;
      hilbert_decode(first, b, pt, py, px);
      const int side_bits = b - lev;
      const uint32_t side = 1u << side_bits;
      pt = (pt >> side_bits) << side_bits;
      py = (py >> side_bits) << side_bits;
      px = (px >> side_bits) << side_bits;
      before = clipped(pt, side, T) * clipped(py, side, Y) * clipped(px, side, X);
    }
  }
  before = block_reduce<kHilbertThreads>(before, s_red,
                                         [](int64_t a, int64_t bb) { return a + bb; });

  // 2. this chunk's points, in curve order.
  const uint32_t chunk = 1u << (3 * m);
  const uint32_t per = chunk >= kHilbertThreads ? chunk / kHilbertThreads : 1u;
  const uint32_t local0 = (uint32_t)tid * per;
  int32_t tok[kMaxPerThread];
  int32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < kMaxPerThread; ++e) {
    tok[e] = -1;
    if ((uint32_t)e < per && local0 + e < chunk) {
      uint32_t pt, py, px;
      hilbert_decode(c * chunk + local0 + e, b, pt, py, px);
      if (pt < (uint32_t)T && py < (uint32_t)Y && px < (uint32_t)X) {
        tok[e] = (int32_t)((pt * (uint32_t)Y + py) * (uint32_t)X + px);
        ++cnt;
      }
    }
  }
  int32_t total;
  int32_t rank = (int32_t)before + block_exclusive_scan<kHilbertThreads>(cnt, s_scan, total);
#pragma unroll
  for (int e = 0; e < kMaxPerThread; ++e) {
    if (tok[e] >= 0 && rank < n_total) {
      perm[rank] = tok[e];
      inv[tok[e]] = rank;
      ++rank;
    }
  }
}

}  // namespace

hipError_t launch_hilbert(int T, int Y, int X, int32_t* perm, int32_t* inv,
                          hipStream_t s) {
  const int mx = max(T, max(Y, X));
  int b = 1;
  while ((1 << b) < mx) ++b;
  const int m = min(b, kMaxChunkBits);
  const unsigned chunks = 1u << (3 * (b - m));
  hipLaunchKernelGGL(hilbert_chunk_kernel, dim3(chunks), dim3(kHilbertThreads),
                     0, s, T, Y, X, b, m, perm, inv);
  return hipGetLastError();
}

}  // namespace fvattn
