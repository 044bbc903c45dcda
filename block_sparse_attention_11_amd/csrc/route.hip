// Routing: block importance from mean-pooled Q/K, Top-p cut with a Top-k
// floor, block mask, kept-block lists, per-head load and density.
//
// Sources: key-block importance is estimated from pooled Q and K, and one
// routing pass gives the mask and the per-head density (PaperDaily FVAttn
// article, method section; aixai.ru FVAttn post, "Sparse-routing frontend");
// Top-p keeps blocks in importance order until the accumulated importance
// reaches p (aixai.ru post, "Top-p vs Top-k"); the Top-k floor keeps at least
// the k most important blocks (PaperDaily article, method section).
// Readings: mean pooling over true rows, importance = softmax over key blocks
// of qbar . kbar / sqrt(d), ranking by (importance desc, index asc), cut at
// the first prefix whose mass is >= p.
//
// Kernels (all fp32 arithmetic):
//   pool_kernel    one workgroup per (block, head, tensor): coalesced 16-byte
//                  row loads, per-lane column sums, LDS reduction.  HBM-bound:
//                  reads Q and K exactly once.
//   score_kernel   z = qbar kbar^T * scale per head, LDS-tiled 64x64 fp32.
//   select_wave_kernel  one wavefront per row for nB <= 2048, four rows per
//                  workgroup: the same arithmetic as select_kernel (so the
//                  same output bytes) with no workgroup barrier.
//   select_kernel  one workgroup per (query block, head): row softmax, bitonic
//                  sort of (P, ~j) keys held in registers (partners in the
//                  same thread swap in place, partners in the wavefront come
//                  by lane shuffle, only the widest stages go through LDS),
//                  workgroup prefix sum, cut, mask row and ascending kept
//                  list via a flag scan.
//   load_kernel    per-head sum of kv_count (exact int64) and density.
#include <math.h>

#include "device_util.h"
#include "internal.h"

namespace fvattn {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kSelectThreads = 256;
constexpr int kScoreTile = 64;
constexpr int kScoreK = 16;

// One 16-byte vector of a row as fp32 values (bf16 widened exactly).
__device__ inline void unpack_vec(const uint4& v, float out[4], const float*) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}

__device__ inline void unpack_vec(const uint4& v, float out[8], const bf16s*) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T>
struct VecWidth { static constexpr int value = 16 / sizeof(T); };

constexpr int kPoolBatch = 8;   // rows one thread has in flight

// Column means of rows r0..r1-1 of one block, in one fixed fp32 order:
// thread (rsub, lane) adds rows r0 + rsub + t * rows_per_pass in ascending t,
// then the rsub partials are added in ascending rsub.  Row r is read from
// src row (GATHER ? index[r] : r); with GATHER it is also stored to out row
// r, so the gather into Hilbert order and the pooling read the rows once.
template <typename T, bool GATHER>
__device__ inline void pool_block(const T* __restrict__ src, T* __restrict__ out,
                                  const int32_t* __restrict__ index,
                                  float* __restrict__ mean, int r0, int r1, int d,
                                  float* red) {
  constexpr int VE = VecWidth<T>::value;
  const int lanes_per_row = d / VE;
  const int rows_per_pass = kPoolThreads / lanes_per_row;
  const int tid = threadIdx.x;
  const int lane = tid % lanes_per_row;
  const int rsub = tid / lanes_per_row;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  if (rsub < rows_per_pass) {
    for (int rb = r0 + rsub; rb < r1; rb += kPoolBatch * rows_per_pass) {
      uint4 raw[kPoolBatch];
#pragma unroll
      for (int t = 0; t < kPoolBatch; ++t) {
        const int r = rb + t * rows_per_pass;
        if (r < r1) {
          const size_t sr = GATHER ? (size_t)index[r] : (size_t)r;
          raw[t] = *reinterpret_cast<const uint4*>(src + sr * d + lane * VE);
        }
      }
#pragma unroll
      for (int t = 0; t < kPoolBatch; ++t) {
        const int r = rb + t * rows_per_pass;
        if (r < r1) {
          if constexpr (GATHER)
            *reinterpret_cast<uint4*>(out + (size_t)r * d + lane * VE) = raw[t];
          float x[VE];
          unpack_vec(raw[t], x, src);
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[e] += x[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) red[tid * VE + e] = acc[e];
  __syncthreads();
  // red[rsub * d + col] holds the partial sum of rows r = rsub (mod passes).
  const int used = min(rows_per_pass, r1 - r0);
  const float inv = 1.0f / (float)(r1 - r0);
  for (int col = tid; col < d; col += kPoolThreads) {
    float s = 0.f;
    for (int rs = 0; rs < used; ++rs) s += red[rs * d + col];
    mean[col] = s * inv;
  }
}

// blockIdx.x = key/query block j, blockIdx.y = head, blockIdx.z = 0 (Q) / 1 (K)
template <typename T>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ qbar,
    float* __restrict__ kbar, int n, int d, int block, int nb) {
  __shared__ float red[kPoolThreads * VecWidth<T>::value];
  const int j = blockIdx.x, h = blockIdx.y;
  const T* src = (blockIdx.z == 0 ? q : k) + (size_t)h * n * d;
  float* dst = (blockIdx.z == 0 ? qbar : kbar) + ((size_t)h * nb + j) * d;
  const int r0 = j * block;
  pool_block<T, false>(src, nullptr, nullptr, dst, r0, min(n, r0 + block), d, red);
}

// Gather into Hilbert order fused with the pooling: blockIdx.x = block j,
// blockIdx.y = head; out[h][r] = src[h][index[r]] for the rows of block j
// and pooled[h][j] = their column means (the same values pool_kernel gives
// for the gathered tensor, bit for bit).
template <typename T>
__global__ __launch_bounds__(kPoolThreads) void permute_pool_kernel(
    const T* __restrict__ src, T* __restrict__ out, const int32_t* __restrict__ index,
    float* __restrict__ pooled, int n, int d, int block, int nb) {
  __shared__ float red[kPoolThreads * VecWidth<T>::value];
  const int j = blockIdx.x, h = blockIdx.y;
  const size_t head = (size_t)h * n * d;
  const int r0 = j * block;
  pool_block<T, true>(src + head, out + head, index, pooled + ((size_t)h * nb + j) * d, r0,
                      min(n, r0 + block), d, red);
}

// z[h][i][j] = scale * sum_c qbar[h][i][c] * kbar[h][j][c]
__global__ __launch_bounds__(256) void score_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar,
    float* __restrict__ z, int nb, int d, float scale) {
  __shared__ float As[kScoreK][kScoreTile + 4];
  __shared__ float Bs[kScoreK][kScoreTile + 4];
  const int h = blockIdx.z;
  const int i0 = blockIdx.y * kScoreTile, j0 = blockIdx.x * kScoreTile;
  const float* A = qbar + (size_t)h * nb * d;
  const float* B = kbar + (size_t)h * nb * d;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;   // 4x4 outputs per thread
  float acc[4][4] = {};
  for (int c0 = 0; c0 < d; c0 += kScoreK) {
    // 64 rows x 16 columns of each operand: 1024 values, 4 per thread.
    for (int e = tid; e < kScoreTile * kScoreK; e += 256) {
      const int r = e / kScoreK, c = e % kScoreK;
      const int ar = i0 + r, br = j0 + r, cc = c0 + c;
      As[c][r] = (ar < nb && cc < d) ? A[(size_t)ar * d + cc] : 0.f;
      Bs[c][r] = (br < nb && cc < d) ? B[(size_t)br * d + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kScoreK; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) a[x] = As[c][ti * 4 + x];
#pragma unroll
      for (int y = 0; y < 4; ++y) b[y] = Bs[c][tj * 4 + y];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = i0 + ti * 4 + x;
    if (i >= nb) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = j0 + tj * 4 + y;
      if (j < nb) z[((size_t)h * nb + i) * nb + j] = acc[x][y] * scale;
    }
  }
}

// One workgroup per row (i = blockIdx.x, h = blockIdx.y).  Dynamic LDS:
// np uint64 sort keys + np floats (prefix sums) + np ints (flags/positions),
// np = next power of two >= nb.
// KP = np / kSelectThreads keys per thread (thread t holds ranks KP*t ..).
template <int KP>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const float* __restrict__ z, int nb, int np, float p, int k_floor,
    uint8_t* __restrict__ mask, int32_t* __restrict__ kv_count,
    int32_t* __restrict__ kv_index) {
  extern __shared__ uint64_t smem[];
  uint64_t* keys = smem;
  float* cum = reinterpret_cast<float*>(keys + np);
  int32_t* flag = reinterpret_cast<int32_t*>(cum + np);
  __shared__ float s_redf[kSelectThreads / kWave];
  __shared__ int32_t s_redi[kSelectThreads / kWave];

  const int i = blockIdx.x, h = blockIdx.y;
  const size_t row = (size_t)h * nb + i;
  const float* zr = z + row * nb;
  const int tid = threadIdx.x;

  // softmax over the row
  float mx = -INFINITY;
  for (int j = tid; j < nb; j += kSelectThreads) mx = fmaxf(mx, zr[j]);
  mx = block_reduce<kSelectThreads>(mx, s_redf, [](float a, float b) { return fmaxf(a, b); });
  float sum = 0.f;
  for (int j = tid; j < nb; j += kSelectThreads) {
    const float e = expf(zr[j] - mx);
    cum[j] = e;
    sum += e;
  }
  // deterministic order: per-thread strided partials, then a fixed tree
  sum = block_reduce<kSelectThreads>(sum, s_redf, [](float a, float b) { return a + b; });
  __syncthreads();                   // cum[] is read across threads below
  uint64_t kr[KP];
#pragma unroll
  for (int e = 0; e < KP; ++e) {
    const int j = KP * tid + e;
    // (P, ~j): P descending, then j ascending; padding (0) sorts last
    kr[e] = j < nb ? ((uint64_t)__float_as_uint(cum[j] / sum) << 32) | (uint64_t)(~(uint32_t)j)
                   : 0;
  }

  // bitonic sort, descending.  A stage pairs rank x with x ^ jj; the lower
  // rank takes the larger key where (x & kk) == 0, the smaller elsewhere.
  // Partners in this thread's registers swap in place, partners in this
  // wavefront come by lane shuffle, others through LDS (one barrier each).
  for (int kk = 2; kk <= np; kk <<= 1) {
    int jj = kk >> 1;
    if (jj >= 64 * KP) {
#pragma unroll
      for (int e = 0; e < KP; ++e) keys[KP * tid + e] = kr[e];
      __syncthreads();
      for (; jj >= 64 * KP; jj >>= 1) {
        for (int x = tid; x < np; x += kSelectThreads) {
          const int y = x ^ jj;
          if (y > x) {
            const uint64_t a = keys[x], b = keys[y];
            const bool desc = (x & kk) == 0;
            if (desc ? (a < b) : (a > b)) {
              keys[x] = b;
              keys[y] = a;
            }
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int e = 0; e < KP; ++e) kr[e] = keys[KP * tid + e];
    }
    for (; jj >= KP; jj >>= 1) {
      const int lanes = jj / KP;       // partner thread tid ^ lanes, same wavefront
#pragma unroll
      for (int e = 0; e < KP; ++e) {
        const int x = KP * tid + e;
        const uint64_t mine = kr[e];
        const uint64_t other = (uint64_t)__shfl_xor((long long)mine, lanes, kWave);
        const bool keep_max = ((x & jj) == 0) == ((x & kk) == 0);
        kr[e] = keep_max ? (mine > other ? mine : other) : (mine < other ? mine : other);
      }
    }
    // in-register stages jr = min(jj, KP/2) .. 1 (compile-time register indices)
#pragma unroll
    for (int jr = KP / 2; jr >= 1; jr >>= 1) {
      if (jr <= jj) {
#pragma unroll
        for (int e = 0; e < KP; ++e) {
          if ((e & jr) == 0) {
            const int x = KP * tid + e;
            const uint64_t a = kr[e], b = kr[e | jr];
            const bool desc = (x & kk) == 0;
            if (desc ? (a < b) : (a > b)) {
              kr[e] = b;
              kr[e | jr] = a;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < KP; ++e) keys[KP * tid + e] = kr[e];
  __syncthreads();

  // inclusive prefix sum of P in ranked order: contiguous per-thread chunks
  const int per = np / kSelectThreads > 0 ? np / kSelectThreads : 1;
  const int c0 = tid * per;
  float run = 0.f;
  for (int e = 0; e < per; ++e) {
    const int x = c0 + e;
    if (x < np) {
      run += __uint_as_float((uint32_t)(keys[x] >> 32));
      cum[x] = run;
    }
  }
  __syncthreads();
  {
    // exclusive scan of the chunk totals (float, fixed order)
    float* tot = reinterpret_cast<float*>(flag);   // reuse as scratch
    tot[tid] = run;
    __syncthreads();
    if (tid == 0) {
      // all prefixes left to right in one thread: base(t) = ((tot[0] + tot[1])
      // + ...) + tot[t-1], the sum each thread would form for itself
      float b = 0.f;
      for (int t = 0; t < kSelectThreads; ++t) {
        const float v = tot[t];
        tot[t] = b;
        b += v;
      }
    }
    __syncthreads();
    const float base = tot[tid];
    __syncthreads();
    for (int e = 0; e < per; ++e) {
      const int x = c0 + e;
      if (x < np) cum[x] += base;
    }
  }
  __syncthreads();

  int n_p = nb;
  if (p < 1.0f) {
    int first = nb;
    for (int x = tid; x < nb; x += kSelectThreads)
      if (cum[x] >= p) { first = min(first, x); }
    first = block_reduce<kSelectThreads>(first, s_redi, [](int a, int b) { return min(a, b); });
    n_p = first < nb ? first + 1 : nb;
  }
  const int n_keep = min(nb, max(n_p, k_floor));

  for (int j = tid; j < nb; j += kSelectThreads) flag[j] = 0;
  __syncthreads();
  for (int x = tid; x < n_keep; x += kSelectThreads)
    flag[~(uint32_t)(keys[x] & 0xffffffffu)] = 1;
  __syncthreads();

  uint8_t* mrow = mask + row * nb;
  for (int j = tid; j < nb; j += kSelectThreads) mrow[j] = (uint8_t)flag[j];
  // ascending compaction: contiguous chunks of j per thread, workgroup scan
  const int perj = (nb + kSelectThreads - 1) / kSelectThreads;
  const int j0 = tid * perj;
  int mine = 0;
  for (int e = 0; e < perj; ++e) {
    const int j = j0 + e;
    if (j < nb) mine += flag[j];
  }
  int total;
  int pos = block_exclusive_scan<kSelectThreads>(mine, s_redi, total);
  int32_t* irow = kv_index + row * nb;
  for (int e = 0; e < perj; ++e) {
    const int j = j0 + e;
    if (j < nb && flag[j]) irow[pos++] = j;
  }
  if (tid == 0) kv_count[row] = n_keep;
}

// One wavefront per row, four rows per workgroup, for np <= 2048 (nB <=
// 2048): the same arithmetic as select_kernel, so the same output bytes, with
// no workgroup barrier.  Virtual thread t of select_kernel's 256 (its row
// max, row-sum partial and prefix chunk) lives in lane t % 64 of this
// wavefront, so lane l holds the sums of t = l, l+64, l+128, l+192 and the
// sorted ranks KW*l .. KW*l + KW - 1, which are select_kernel's prefix chunks
// 4l .. 4l+3 (np/256 ranks each).  The bitonic network runs in registers
// (partners within a lane) and by lane shuffles (partners in other lanes).
// Per wavefront LDS: the row's exponentials (np floats) and the kept flags
// (np bytes).
constexpr int kWaveRows = 4;

template <int KW>
__global__ __launch_bounds__(kWave * kWaveRows) void select_wave_kernel(
    const float* __restrict__ z, int nb, int rows, float p, int k_floor,
    uint8_t* __restrict__ mask, int32_t* __restrict__ kv_count,
    int32_t* __restrict__ kv_index) {
  constexpr int NP = KW * kWave;                 // padded row length (power of two)
  constexpr int PER = NP / kSelectThreads;       // select_kernel's prefix chunk
  static_assert(PER * 4 == KW, "four prefix chunks per lane");
  __shared__ float s_e[kWaveRows][NP];
  __shared__ uint8_t s_flag[kWaveRows][NP];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int row = blockIdx.x * kWaveRows + wv;
  if (row >= rows) return;                       // whole wavefront; no barrier below
  const float* zr = z + (size_t)row * nb;
  float* e_row = s_e[wv];
  uint8_t* flag = s_flag[wv];

  // row max (order-free), then the row sum in select_kernel's order: virtual
  // thread t = 64w + l adds j = t, t + 256, ... in ascending j; each
  // wavefront of virtual threads reduces by an xor butterfly; the four
  // results add in wavefront order
  float mx = -INFINITY;
  for (int j = lane; j < nb; j += kWave) mx = fmaxf(mx, zr[j]);
  mx = wave_max(mx);
  float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    for (int j = kWave * w + lane; j < nb; j += kSelectThreads) {
      const float e = expf(zr[j] - mx);
      e_row[j] = e;
      part[w] += e;
    }
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) part[w] += __shfl_xor(part[w], off, kWave);
  }
  const float sum = ((part[0] + part[1]) + part[2]) + part[3];

  uint64_t kr[KW];
#pragma unroll
  for (int e = 0; e < KW; ++e) {
    const int j = KW * lane + e;
    kr[e] = j < nb ? ((uint64_t)__float_as_uint(e_row[j] / sum) << 32) | (uint64_t)(~(uint32_t)j)
                   : 0;
  }
  // bitonic sort, descending.  Keys are unique, so the result is the order
  // select_kernel produces.  Ranks x = KW*lane + e; a stage (kk, jj) pairs x
  // with x ^ jj and the pair's lower rank takes the larger key where
  // (x & kk) == 0.  kk <= KW: lane-local stages, unrolled (the direction is a
  // constant, or the lane's parity at kk = KW); kk > KW: partners in other
  // lanes (jj >= KW, by shuffle) or in this lane (jj < KW), the direction a
  // per-lane constant of the stage.
  auto ce = [&](int e0, int e1, bool desc) {
    // order kr[e0] >= kr[e1] when desc, else kr[e0] <= kr[e1]
    const uint64_t a = kr[e0], b = kr[e1];
    const bool sw = (a < b) == desc;
    kr[e0] = sw ? b : a;
    kr[e1] = sw ? a : b;
  };
#pragma unroll
  for (int kk = 2; kk <= KW; kk <<= 1) {
    const bool lane_desc = kk < KW ? true : (lane & 1) == 0;
#pragma unroll
    for (int jr = kk >> 1; jr >= 1; jr >>= 1) {
#pragma unroll
      for (int e = 0; e < KW; ++e)
        if ((e & jr) == 0) ce(e, e | jr, kk < KW ? (e & kk) == 0 : lane_desc);
    }
  }
#pragma unroll 1
  for (int kk = 2 * KW; kk <= NP; kk <<= 1) {
    const bool desc = ((KW * lane) & kk) == 0;
#pragma unroll 1
    for (int jj = kk >> 1; jj >= KW; jj >>= 1) {
      const int lanes = jj / KW;
      // the lower rank of each pair keeps the larger key where desc
      const bool keep_max = (((KW * lane) & jj) == 0) == desc;
#pragma unroll
      for (int e = 0; e < KW; ++e) {
        const uint64_t mine = kr[e];
        const uint64_t other = (uint64_t)__shfl_xor((long long)mine, lanes, kWave);
        kr[e] = ((other > mine) == keep_max) ? other : mine;
      }
    }
#pragma unroll
    for (int jr = KW / 2; jr >= 1; jr >>= 1) {
#pragma unroll
      for (int e = 0; e < KW; ++e)
        if ((e & jr) == 0) ce(e, e | jr, desc);
    }
  }

  // prefix sums in select_kernel's order: PER ranks per chunk summed in
  // order, chunk bases accumulated left to right over all 256 chunks (the
  // chunks of lane 0, then lane 1, ...), carried from lane to lane
  float cum[KW], tot[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      run += __uint_as_float((uint32_t)(kr[PER * c + e] >> 32));
      cum[PER * c + e] = run;
    }
    tot[c] = run;
  }
  float base[4] = {0.f, 0.f, 0.f, 0.f};
  {
    float b = 0.f;                                 // wave-uniform running base
#pragma unroll 1
    for (int l = 0; l < kWave; ++l) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float t = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tot[c]), l));
        if (lane == l) base[c] = b;
        b += t;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int e = 0; e < PER; ++e) cum[PER * c + e] += base[c];
  }

  int n_p = nb;
  if (p < 1.0f) {
    int first = nb;
#pragma unroll
    for (int e = KW - 1; e >= 0; --e) {
      const int x = KW * lane + e;
      if (x < nb && cum[e] >= p) first = x;
    }
    first = wave_min(first);
    n_p = first < nb ? first + 1 : nb;
  }
  const int n_keep = min(nb, max(n_p, k_floor));

  for (int j = lane; j < NP; j += kWave) flag[j] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int e = 0; e < KW; ++e)
    if (KW * lane + e < n_keep) flag[~(uint32_t)(kr[e] & 0xffffffffu)] = 1;
  __builtin_amdgcn_wave_barrier();

  uint8_t* mrow = mask + (size_t)row * nb;
  for (int j = lane; j < nb; j += kWave) mrow[j] = flag[j];
  // ascending compaction: contiguous chunks of j per lane, wavefront scan
  const int perj = (nb + kWave - 1) / kWave;
  const int j0 = lane * perj;
  int mine = 0;
  for (int e = 0; e < perj; ++e) {
    const int j = j0 + e;
    if (j < nb) mine += flag[j];
  }
  int pos = wave_inclusive_scan(mine) - mine;
  int32_t* irow = kv_index + (size_t)row * nb;
  for (int e = 0; e < perj; ++e) {
    const int j = j0 + e;
    if (j < nb && flag[j]) irow[pos++] = j;
  }
  if (lane == 0) kv_count[row] = n_keep;
}

__global__ __launch_bounds__(256) void load_kernel(
    const int32_t* __restrict__ kv_count, int nb, int64_t* __restrict__ head_load,
    float* __restrict__ head_density) {
  __shared__ int64_t s_red[256 / kWave];
  const int h = blockIdx.x;
  int64_t s = 0;
  for (int i = threadIdx.x; i < nb; i += 256) s += kv_count[(size_t)h * nb + i];
  s = block_reduce<256>(s, s_red, [](int64_t a, int64_t b) { return a + b; });
  if (threadIdx.x == 0) {
    head_load[h] = s;
    head_density[h] = (float)((double)s / ((double)nb * (double)nb));
  }
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

size_t route_workspace_bytes(int heads, int n, int d, int block) {
  const size_t nb = ((size_t)n + block - 1) / block;
  const size_t pooled = align_up(sizeof(float) * (size_t)heads * nb * d, 256);
  const size_t scores = align_up(sizeof(float) * (size_t)heads * nb * nb, 256);
  return 2 * pooled + scores;
}

RouteWorkspace route_carve(void* ws, int heads, int n, int d, int block) {
  const size_t nb = ((size_t)n + block - 1) / block;
  const size_t pooled = align_up(sizeof(float) * (size_t)heads * nb * d, 256);
  char* base = static_cast<char*>(ws);
  RouteWorkspace w;
  w.qbar = reinterpret_cast<float*>(base);
  w.kbar = reinterpret_cast<float*>(base + pooled);
  w.z = reinterpret_cast<float*>(base + 2 * pooled);
  return w;
}

hipError_t launch_head_load(const int32_t* kv_count, int heads, int nb, int64_t* head_load,
                            float* head_density, hipStream_t s) {
  hipLaunchKernelGGL(load_kernel, dim3(heads), dim3(256), 0, s, kv_count, nb, head_load,
                     head_density);
  return hipGetLastError();
}

hipError_t launch_permute_pool(const void* src, void* dst, const int32_t* index, bool bf16,
                               int heads, int n, int d, int block, float* pooled,
                               hipStream_t s) {
  const int nb = (n + block - 1) / block;
  if (bf16) {
    hipLaunchKernelGGL(permute_pool_kernel<bf16s>, dim3(nb, heads), dim3(kPoolThreads), 0, s,
                       (const bf16s*)src, (bf16s*)dst, index, pooled, n, d, block, nb);
  } else {
    hipLaunchKernelGGL(permute_pool_kernel<float>, dim3(nb, heads), dim3(kPoolThreads), 0, s,
                       (const float*)src, (float*)dst, index, pooled, n, d, block, nb);
  }
  return hipGetLastError();
}

hipError_t launch_route(const void* q, const void* k, bool bf16, int heads,
                        int n, int d, int block, float p, int k_floor,
                        uint8_t* mask, int32_t* kv_count, int32_t* kv_index,
                        int64_t* head_load, float* head_density,
                        const RouteWorkspace& ws, hipStream_t s) {
  const int nb = (n + block - 1) / block;
  if (bf16) {
    hipLaunchKernelGGL(pool_kernel<bf16s>, dim3(nb, heads, 2),
                       dim3(kPoolThreads), 0, s, (const bf16s*)q,
                       (const bf16s*)k, ws.qbar, ws.kbar, n, d, block, nb);
  } else {
    hipLaunchKernelGGL(pool_kernel<float>, dim3(nb, heads, 2), dim3(kPoolThreads),
                       0, s, (const float*)q, (const float*)k, ws.qbar, ws.kbar, n,
                       d, block, nb);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_route_pooled(ws.qbar, ws.kbar, heads, n, d, block, p, k_floor, mask,
                             kv_count, kv_index, head_load, head_density, ws, s);
}

hipError_t launch_route_pooled(const float* qbar, const float* kbar, int heads, int n,
                               int d, int block, float p, int k_floor, uint8_t* mask,
                               int32_t* kv_count, int32_t* kv_index, int64_t* head_load,
                               float* head_density, const RouteWorkspace& ws,
                               hipStream_t s) {
  const int nb = (n + block - 1) / block;
  const unsigned tiles = (unsigned)((nb + kScoreTile - 1) / kScoreTile);
  hipLaunchKernelGGL(score_kernel, dim3(tiles, tiles, heads), dim3(256), 0, s,
                     qbar, kbar, ws.z, nb, d, 1.0f / sqrtf((float)d));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int np = 1;
  while (np < nb) np <<= 1;
  if (np < kSelectThreads) np = kSelectThreads;
  if (np <= 2048) {
    // one wavefront per row (same output bytes as select_kernel)
    const int rows = heads * nb;
    const dim3 wgrid((rows + kWaveRows - 1) / kWaveRows);
    const dim3 wblock(kWave * kWaveRows);
    switch (np) {
      case 256:
        hipLaunchKernelGGL(select_wave_kernel<4>, wgrid, wblock, 0, s, ws.z, nb, rows, p,
                           k_floor, mask, kv_count, kv_index);
        break;
      case 512:
        hipLaunchKernelGGL(select_wave_kernel<8>, wgrid, wblock, 0, s, ws.z, nb, rows, p,
                           k_floor, mask, kv_count, kv_index);
        break;
      case 1024:
        hipLaunchKernelGGL(select_wave_kernel<16>, wgrid, wblock, 0, s, ws.z, nb, rows, p,
                           k_floor, mask, kv_count, kv_index);
        break;
      default:
        hipLaunchKernelGGL(select_wave_kernel<32>, wgrid, wblock, 0, s, ws.z, nb, rows, p,
                           k_floor, mask, kv_count, kv_index);
        break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_head_load(kv_count, heads, nb, head_load, head_density, s);
  }
  const size_t lds = (size_t)np * (sizeof(uint64_t) + sizeof(float) + sizeof(int32_t));
  const dim3 grid(nb, heads);
  switch (np / kSelectThreads) {
    case 1:
      hipLaunchKernelGGL(select_kernel<1>, grid, dim3(kSelectThreads), lds, s, ws.z, nb, np, p,
                         k_floor, mask, kv_count, kv_index);
      break;
    case 2:
      hipLaunchKernelGGL(select_kernel<2>, grid, dim3(kSelectThreads), lds, s, ws.z, nb, np, p,
                         k_floor, mask, kv_count, kv_index);
      break;
    case 4:
      hipLaunchKernelGGL(select_kernel<4>, grid, dim3(kSelectThreads), lds, s, ws.z, nb, np, p,
                         k_floor, mask, kv_count, kv_index);
      break;
    case 8:
      hipLaunchKernelGGL(select_kernel<8>, grid, dim3(kSelectThreads), lds, s, ws.z, nb, np, p,
                         k_floor, mask, kv_count, kv_index);
      break;
    default:                            // nB <= 4096: at most 16 keys per thread
      hipLaunchKernelGGL(select_kernel<16>, grid, dim3(kSelectThreads), lds, s, ws.z, nb, np,
                         p, k_floor, mask, kv_count, kv_index);
      break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_head_load(kv_count, heads, nb, head_load, head_density, s);
}

}  // namespace fvattn
