// Block-sparse attention over the kept key blocks.
//
// Source: sparse attention computes only the (query block, key block) pairs
// the routing keeps (aixai.ru FVAttn post, "What is sparse attention in video
// transformers"; arXiv abstract on the mlsanity.com index page).  For tile
// (h, i): O_i = softmax(Q_i K_S^T * scale) V_S over the rows S of the kept
// blocks, evaluated block by block with an online (running max / running
// sum) softmax in fp32.
//
// The MFMA formulation, shared by the three bf16 kernels (storage bf16,
// v_mfma_f32_32x32x16_bf16, each wavefront owns 32 queries).  Everything is
// computed transposed,
//       S^T[key][q] = K Q^T      (A = K rows from LDS, B = Q from registers)
//       O^T[d][q]  += V^T P^T    (A = V^T rows from LDS, B = P from registers)
//   so in both accumulators lane l holds query l%32: the row max and row sum
//   need one exchange with lane l^32, the rescale is a per-lane scalar, and
//   the S^T accumulator registers are already the B operand of the PV product
//   (the 16-key chunks are taken in the order the accumulator layout gives;
//   V^T is read from LDS in that same order).  K is staged in LDS row-major
//   with an XOR swizzle of its 16-byte chunks, V transposed with an XOR
//   swizzle (of 8-byte units in attn_mfma_kernel, of 16-byte chunks in the
//   two copy kernels), conflict-free for the MFMA reads.  The softmax runs in
//   the exp2 domain with scale*log2(e) folded into one FMA per score; P is
//   rounded to bf16 (round to nearest even) for the PV product.
//
// Kernels:
//
// attn_mfma_tile_kernel<D, BLK, G, HK>  the default: persistent workgroups of
//   G consecutive q-blocks (G = 2, or 3) that walk the union of their kept
//   lists, with K and V^T key-block tiles copied into LDS by buffer loads
//   straight to LDS, double buffered, one barrier per key block, and
//   run-time tile claims.
// attn_mfma_dma_kernel<D, BLK>  the same copies for one q-block per
//   workgroup (BLK/32 wavefronts).
// attn_mfma_kernel<D, BLK>  one q-block per workgroup, V in row layout,
//   staged through registers.
// attn_simple_kernel<T, DMAX>  plain fp32 VALU reference kernel for every
//   other shape (fp32 inputs, small head dims, odd block sizes): one thread
//   per query row, K/V staged through LDS in chunks of 32 rows.
//
// All run either persistently (workgroup w walks its LPT list) or as a
// head-major grid (one workgroup per tile), and write per-workgroup
// timestamps (s_memrealtime, 100 MHz) plus the HW_ID / XCC_ID registers.
#include <math.h>

#include "device_util.h"
#include "internal.h"

namespace fvattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// hardware register ids for s_getreg (gfx9.4+): HW_ID and XCC_ID, 32 bits
constexpr int kGetregHwId = (31 << 11) | 4;
constexpr int kGetregXccId = (31 << 11) | 20;

__device__ inline void stamp_start(uint64_t& t0) {
  t0 = __builtin_amdgcn_s_memrealtime();
}

__device__ inline void stamp_end(uint64_t* timing, int w, uint64_t t0) {
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  timing[4 * (size_t)w + 0] = t0;
  timing[4 * (size_t)w + 1] = t1;
  timing[4 * (size_t)w + 2] = (uint64_t)__builtin_amdgcn_s_getreg(kGetregHwId);
  timing[4 * (size_t)w + 3] = (uint64_t)__builtin_amdgcn_s_getreg(kGetregXccId);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite or +-inf).
__device__ inline uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr bf16x2 kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T>
__device__ inline float load_elem(const T* p);
template <>
__device__ inline float load_elem<float>(const float* p) { return *p; }
template <>
__device__ inline float load_elem<bf16s>(const bf16s* p) {
  return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
}

template <typename T>
__device__ inline void store_elem(T* p, float v);
template <>
__device__ inline void store_elem<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void store_elem<bf16s>(bf16s* p, float v) {
  *reinterpret_cast<uint16_t*>(p) = (uint16_t)bf16_bits(v);
}

// Marks a uniform branch body as not to be speculated: without it the
// compiler turns rarely taken branches (the tail-block key mask, the lazy
// rescale) into unconditional selects executed on every block.
__device__ inline void keep_branch() { asm volatile(""); }

// max of v over lanes l and l ^ 32 (the two halves of a wavefront), with one
// VALU lane swap instead of a round trip through LDS
__device__ inline float max_with_other_half(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                   false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// ---------------------------------------------------------------------------
// Plain fp32 kernel.
// ---------------------------------------------------------------------------
constexpr int kSimpleThreads = 256;
constexpr float kRescaleSlack = 8.0f;

// the row of o that result row r goes to: the caller's scatter (for instance
// back to token order) or r itself
__device__ inline int out_row(const AttnArgs& a, int r) {
  return a.out_rows ? a.out_rows[r] : r;
}
constexpr int kSimpleChunk = 32;

template <typename T, int DMAX, bool PERSIST>
__global__ __launch_bounds__(kSimpleThreads) void attn_simple_kernel(AttnArgs a) {
  __shared__ float Ks[kSimpleChunk][DMAX];
  __shared__ float Vs[kSimpleChunk][DMAX];
  const int tid = threadIdx.x;
  const int n = a.n, d = a.d, blk = a.block, nb = a.nb;
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  T* O = static_cast<T*>(a.o);
  uint64_t t0 = 0;
  if (PERSIST && a.timing && tid == 0) stamp_start(t0);

  int beg = blockIdx.x, end = blockIdx.x + 1;
  if (PERSIST) {
    beg = a.worker_offsets[blockIdx.x];
    end = a.worker_offsets[blockIdx.x + 1];
  }
  for (int it = beg; it < end; ++it) {
    const int tile = PERSIST ? a.worker_tiles[it] : it;
    const int h = tile / a.tiles_per_head;
    const int gm = tile - h * a.tiles_per_head;
    for (int i = gm * a.group; i < min(nb, (gm + 1) * a.group); ++i) {
    const int r = i * blk + tid;
    const bool active = tid < blk && r < n;
    const size_t hb = (size_t)h * n;
    float qv[DMAX], acc[DMAX];
#pragma unroll
    for (int c = 0; c < DMAX; ++c) {
      qv[c] = (active && c < d) ? load_elem(Q + (hb + r) * d + c) * a.scale_log2 : 0.f;
      acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int cnt = min(a.kv_count[(size_t)h * nb + i], nb);
    const int32_t* idx = a.kv_index + ((size_t)h * nb + i) * nb;
    for (int jj = 0; jj < cnt; ++jj) {
      const int j = idx[jj];
      if (j < 0 || j >= nb) continue;          // malformed list entry: skip
      const int r0 = j * blk, r1 = min(n, r0 + blk);
      for (int kc = r0; kc < r1; kc += kSimpleChunk) {
        __syncthreads();
        for (int e = tid; e < kSimpleChunk * DMAX; e += kSimpleThreads) {
          const int kr = e / DMAX, c = e % DMAX;
          const int row = kc + kr;
          const bool ok = row < r1 && c < d;
          Ks[kr][c] = ok ? load_elem(K + (hb + row) * d + c) : 0.f;
          const int kr0 = row - r0;
          const size_t vi = a.v_tiles
              ? (((size_t)h * nb + j) * d + c) * blk + vt_pos(kr0)
              : (hb + row) * d + c;
          Vs[kr][c] = ok ? load_elem(V + vi) : 0.f;
        }
        __syncthreads();
        if (active) {
          const int rows = min(kSimpleChunk, r1 - kc);
          for (int kr = 0; kr < rows; ++kr) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < DMAX; ++c) s = fmaf(qv[c], Ks[kr][c], s);
            const float mn = fmaxf(m, s);
            const float corr = mn == -INFINITY ? 1.f : exp2f(m - mn);
            const float pr = mn == -INFINITY ? 0.f : exp2f(s - mn);
            l = l * corr + pr;
#pragma unroll
            for (int c = 0; c < DMAX; ++c) acc[c] = fmaf(pr, Vs[kr][c], acc[c] * corr);
            m = mn;
          }
        }
      }
    }
    if (active) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int c = 0; c < DMAX; ++c)
        if (c < d) store_elem(O + (hb + out_row(a, r)) * d + c, acc[c] * inv);
    }
    }  // q-blocks of the tile
  }
  if (PERSIST && a.timing) {
    __syncthreads();
    if (tid == 0) stamp_end(a.timing, blockIdx.x, t0);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.
// ---------------------------------------------------------------------------
template <int D, int BLK>
struct MfmaShape {
  static constexpr int kWaves = BLK / 32;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kChunksPerRow = D / 8;      // 16-byte chunks of a K row
  static constexpr int kUnitsPerRow = BLK / 4;     // 8-byte units of a V^T row
  static constexpr int kKChunksPerThread = BLK * kChunksPerRow / kThreads;
  static constexpr int kVUnitsPerThread = (BLK / 4) * (D / 8) / kThreads;
  static_assert(kKChunksPerThread * kThreads == BLK * kChunksPerRow, "K staging");
  static_assert(kVUnitsPerThread * kThreads == (BLK / 4) * (D / 8), "V staging");
};

// byte offset of 16-byte chunk c of K row r
template <int D>
__device__ inline uint32_t k_off(int r, int c) {
  constexpr int CPR = D / 8;
  return (uint32_t)(r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4));
}

// byte offset of 8-byte unit u (keys 4u..4u+3) of V^T row dd
template <int BLK>
__device__ inline uint32_t v_off(int dd, int u) {
  constexpr int UPR = BLK / 4;
  return (uint32_t)(dd * (2 * BLK) + ((u ^ (dd & (UPR - 1))) << 3));
}

template <int D, int BLK, bool PERSIST>
__global__ __launch_bounds__(2 * BLK) void attn_mfma_kernel(AttnArgs a) {
  using S = MfmaShape<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint8_t Ks[BLK * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[D * BLK * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;      // query within the wavefront's 32
  const int g = lane >> 5;        // which half of the K dimension this lane feeds
  const int n = a.n, nb = a.nb;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  uint16_t* O = static_cast<uint16_t*>(a.o);
  const float sl2 = a.scale_log2;

  uint64_t t0 = 0;
  if (PERSIST && a.timing && tid == 0) stamp_start(t0);

  int beg = blockIdx.x, end = blockIdx.x + 1;
  if (PERSIST) {
    beg = a.worker_offsets[blockIdx.x];
    end = a.worker_offsets[blockIdx.x + 1];
  }
  for (int it = beg; it < end; ++it) {
    const int tile = PERSIST ? a.worker_tiles[it] : it;
    const int h = tile / a.tiles_per_head;
    const int gm = tile - h * a.tiles_per_head;
    for (int i = gm * a.group; i < min(nb, (gm + 1) * a.group); ++i) {
    const size_t hb = (size_t)h * n;
    const int qrow = i * BLK + wave * 32 + col;
    const bool qvalid = qrow < n;

    // Q^T operand: lane (col, g) holds Q[qrow][16*kk + 8*g .. +7]
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid)
        w = *reinterpret_cast<const u32x4*>(Q + (hb + qrow) * D + 16 * kk + 8 * g);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
    f32x16 acc_o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[dt][e] = 0.f;
    float m_run = -INFINITY;   // running max, log2-scaled units
    float l_run = 0.f;         // running sum over this lane's half of the keys

    const int cnt = min(a.kv_count[(size_t)h * nb + i], nb);
    const int32_t* idx = a.kv_index + ((size_t)h * nb + i) * nb;
    for (int jj = 0; jj < cnt; ++jj) {
      const int j = __builtin_amdgcn_readfirstlane(idx[jj]);
      if (j < 0 || j >= nb) continue;          // malformed list entry: skip
      const int r0 = j * BLK;
      __syncthreads();
      // stage K rows (swizzled 16-byte chunks)
#pragma unroll
      for (int e = 0; e < S::kKChunksPerThread; ++e) {
        const int gidx = tid + e * S::kThreads;
        const int r = gidx / S::kChunksPerRow;
        const int c = gidx % S::kChunksPerRow;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (r0 + r < n) w = *reinterpret_cast<const u32x4*>(K + (hb + r0 + r) * D + 8 * c);
        *reinterpret_cast<u32x4*>(Ks + k_off<D>(r, c)) = w;
      }
      // stage V transposed: a unit is 4 keys x 8 columns
#pragma unroll
      for (int e = 0; e < S::kVUnitsPerThread; ++e) {
        const int gidx = tid + e * S::kThreads;
        const int c8 = gidx % (D / 8);
        const int kq = gidx / (D / 8);
        u32x4 rows[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = r0 + 4 * kq + x;
          rows[x] = u32x4{0u, 0u, 0u, 0u};
          if (r < n) rows[x] = *reinterpret_cast<const u32x4*>(V + (hb + r) * D + 8 * c8);
        }
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int wsel = dd >> 1;
          const int sh = (dd & 1) * 16;
          const uint32_t k0 = (rows[0][wsel] >> sh) & 0xffffu;
          const uint32_t k1 = (rows[1][wsel] >> sh) & 0xffffu;
          const uint32_t k2 = (rows[2][wsel] >> sh) & 0xffffu;
          const uint32_t k3 = (rows[3][wsel] >> sh) & 0xffffu;
          const u32x2 pk = {k0 | (k1 << 16), k2 | (k3 << 16)};
          *reinterpret_cast<u32x2*>(Vt + v_off<BLK>(8 * c8 + dd, kq)) = pk;
        }
      }
      __syncthreads();

      // S^T = K Q^T: tile kt covers keys 32*kt .. 32*kt+31 of the block
      f32x16 s[BLK / 32];
#pragma unroll
      for (int kt = 0; kt < BLK / 32; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(Ks + k_off<D>(32 * kt + col, 2 * kk + g));
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                          qf[kk], s[kt], 0, 0, 0);
        }
      }
      // accumulator layout: s[kt][e] is key 32*kt + 8*(e/4) + 4*g + e%4
      if (r0 + BLK > n) {
      keep_branch();
#pragma unroll
        for (int kt = 0; kt < BLK / 32; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = r0 + 32 * kt + 8 * (e >> 2) + 4 * g + (e & 3);
            if (key >= n) s[kt][e] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < BLK / 32; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescale: the reference max m_run only moves when this block's
      // max exceeds it by more than kRescaleSlack (log2 units), so the
      // exponentials stay below 2^kRescaleSlack and O / l are rescaled about
      // once per tile instead of once per block.  Any m_run gives the same
      // softmax; only rounding differs.
      const float mxs = mx * sl2;
      const bool grow = mxs > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
      keep_branch();
        const float m_new = grow ? mxs : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc_o[dt][e] *= alpha;
      }
      // every score of this row may be masked only if m_run is still -inf
      const float m_sub = m_run == -INFINITY ? 0.f : m_run;

      // P = exp2(S * sl2 - m), rounded to bf16 in accumulator order
      uint32_t pk[BLK / 32][8];
#pragma unroll
      for (int kt = 0; kt < BLK / 32; ++kt)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][e], sl2, -m_sub));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][e + 1], sl2, -m_sub));
          l_run += p0 + p1;
          pk[kt][e >> 1] = pack_bf16x2(p0, p1);
        }

      // O^T += V^T P^T over 16-key chunks c; chunk c uses accumulator
      // registers 8*(c%2) .. +7 of tile c/2 = keys 16c + 8*(e/4) + 4g + e%4.
#pragma unroll
      for (int c = 0; c < BLK / 16; ++c) {
        const u32x4 pb = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1],
                          pk[c >> 1][4 * (c & 1) + 2], pk[c >> 1][4 * (c & 1) + 3]};
        const bf16x8 bop = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int dd = 32 * dt + col;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(Vt + v_off<BLK>(dd, 4 * c + g));
          const u32x2 hi = *reinterpret_cast<const u32x2*>(Vt + v_off<BLK>(dd, 4 * c + 2 + g));
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                              bop, acc_o[dt], 0, 0, 0);
        }
      }
    }

    // normalise and store: acc_o[dt][e] is column d = 32dt + 8(e/4) + 4g + e%4
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qvalid) {
      uint16_t* orow = O + (hb + out_row(a, qrow)) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * dt + 8 * r4 + 4 * g;
          const u32x2 w = {pack_bf16x2(acc_o[dt][4 * r4 + 0] * inv, acc_o[dt][4 * r4 + 1] * inv),
                           pack_bf16x2(acc_o[dt][4 * r4 + 2] * inv, acc_o[dt][4 * r4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
    }
    }  // q-blocks of the tile
  }
  if (PERSIST && a.timing) {
    __syncthreads();
    if (tid == 0) stamp_end(a.timing, blockIdx.x, t0);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel fed by LDS DMA, for V stored as transposed key-block tiles
// ([heads][nb][d][block], see launch_pack_v).  K rows and V^T tiles go from
// HBM/L2 straight into LDS with buffer_load ... lds (no staging registers);
// out-of-range K rows of the short last block read as zero through the
// buffer descriptor's size.  Per key block three barriers order the work:
//   A: K_j has landed and every wave is done with V_{j-1}  -> start V_j DMA
//      S_j = K_j Q^T
//   B: every wave is done with K_j                         -> start K_{j+1} DMA
//      softmax of S_j
//   C: V_j has landed
//      O += V_j^T P_j^T
// so V_j streams in during S_j and the softmax, and K_{j+1} during the
// softmax and the PV product; two workgroups per CU cover the rest.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate for gfx9: wait until at most N vector-memory loads are
// outstanding (exp and lgkm counters left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS reads are complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// vector-memory loads, so LDS-DMA copies keep streaming across it; callers
// wait for the copies they need with wait_vmcnt.  The memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// V^T tiles in LDS: 16-byte chunk c of row dd sits at chunk position
// c ^ vt_swz(dd).  A lane of the P.V MFMA reads chunk 2*cb + g of rows
// 32*dt + col; the XOR term uses the row bits that select 16-byte bank groups
// inside 256 bytes, so each 16 lanes read 16 distinct bank groups.
template <int BLK>
__device__ inline int vt_swz(int dd) {
  constexpr int CPR = BLK / 8;                  // 16-byte chunks of a V^T row
  constexpr int RP = BLK >= 128 ? 1 : 128 / BLK; // rows per 256 bytes
  return (dd / RP) & (CPR - 1);
}
template <int D, int BLK>
__device__ inline uint32_t vt_off(int dd, int chunk) {
  return (uint32_t)(dd * (2 * BLK) + ((chunk ^ vt_swz<BLK>(dd)) << 4));
}

// Buffer descriptor over head h of a tensor whose heads lie head_bytes apart
// (head_bytes < 2^32).  Loads through it take their whole byte offset in the
// per-lane offset operand, which the hardware range check covers: offsets at
// or past head_bytes read as zero, so the rows past the end of a head (the
// short last block) never touch memory outside it, and no tensor size limit
// comes from 32-bit offsets beyond the size of one head.
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int h, uint32_t head_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint8_t*>(base) + (size_t)h * head_bytes), (short)0,
      (int)head_bytes, 0x00020000);
}

// read-only table entry through the scalar cache (the tables are not written
// while the kernel runs and the index is wave-uniform)
__device__ inline int32_t ld_uniform(const int32_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(p));
}

template <int D, int BLK, bool PERSIST>
__global__ __launch_bounds__(2 * BLK, 2) void attn_mfma_dma_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer descriptors exist only in the device pass
  using S = MfmaShape<D, BLK>;
  constexpr int NW = S::kWaves;
  constexpr int CPRK = D / 8;                 // 16-byte chunks per K row
  constexpr int CPRV = BLK / 8;               // 16-byte chunks per V^T row
  constexpr int KDMA = BLK * CPRK / (64 * NW);   // DMA instructions per wave, K
  constexpr int VDMA = D * CPRV / (64 * NW);     // and V
  static_assert(KDMA * 64 * NW == BLK * CPRK && VDMA * 64 * NW == D * CPRV, "DMA split");
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[BLK * D * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs[D * BLK * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int g = lane >> 5;
  const int n = a.n, nb = a.nb;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  uint16_t* O = static_cast<uint16_t*>(a.o);
  const float sl2 = a.scale_log2;
  // one descriptor per head (head_rsrc): K rows past the end of a head read
  // as zero and the score mask removes them
  const uint32_t kbytes = (uint32_t)((size_t)n * D * 2);
  const uint32_t vbytes = (uint32_t)((size_t)nb * D * BLK * 2);

  // per-lane DMA source offsets inside one block (bytes), fixed for the kernel
  uint32_t koff[KDMA], voff[VDMA];
#pragma unroll
  for (int x = 0; x < KDMA; ++x) {
    const int P = (x * NW + wave) * 64 + lane;           // LDS chunk this lane fills
    const int r = P / CPRK, pc = P % CPRK;
    koff[x] = (uint32_t)(r * D * 2 + (pc ^ (r & (CPRK - 1))) * 16);
  }
#pragma unroll
  for (int x = 0; x < VDMA; ++x) {
    const int P = (x * NW + wave) * 64 + lane;
    const int dd = P / CPRV, pc = P % CPRV;
    voff[x] = (uint32_t)(dd * BLK * 2 + (pc ^ vt_swz<BLK>(dd)) * 16);
  }
  auto dma_k = [&](int h, int j) {
    const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k, h, kbytes);
    const uint32_t base = (uint32_t)j * (BLK * D * 2);
#pragma unroll
    for (int x = 0; x < KDMA; ++x)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krs, (lds_void*)(Ks + (x * NW + wave) * 1024), 16, base + koff[x], 0, 0, 0);
  };
  auto dma_v = [&](int h, int j) {
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v, h, vbytes);
    const uint32_t base = (uint32_t)j * (D * BLK * 2);
#pragma unroll
    for (int x = 0; x < VDMA; ++x)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, (lds_void*)(Vs + (x * NW + wave) * 1024), 16, base + voff[x], 0, 0, 0);
  };

  uint64_t t0 = 0;
  if (PERSIST && a.timing && tid == 0) stamp_start(t0);

  int beg = blockIdx.x, end = blockIdx.x + 1;
  if (PERSIST) {
    beg = ld_uniform(a.worker_offsets + blockIdx.x);
    end = ld_uniform(a.worker_offsets + blockIdx.x + 1);
  }
  // tile id, its kept count and list; entries outside [0, nB) are clamped
  auto tile_at = [&](int it) {
    return PERSIST ? ld_uniform(a.worker_tiles + it) : it;
  };
  auto count_of = [&](int tile) { return min(ld_uniform(a.kv_count + tile), nb); };
  auto block_of = [&](int tile, int jj) {
    return min(max(ld_uniform(a.kv_index + (size_t)tile * nb + jj), 0), nb - 1);
  };
  auto zero_rows = [&](int tile) {   // a tile with no kept block
    const int hh = tile / nb, ii = tile - hh * nb;
    const int qr = ii * BLK + wave * 32 + col;
    if (qr < n) {
      uint16_t* orow = O + ((size_t)hh * n + out_row(a, qr)) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * r4 + 4 * g) = u32x2{0u, 0u};
    }
  };
  // first non-empty tile at or after it (zero-filling the empty ones)
  auto advance = [&](int it, int& tile, int& cnt) {
    while (it < end) {
      tile = tile_at(it);
      cnt = count_of(tile);
      if (cnt > 0) break;
      zero_rows(tile);
      ++it;
    }
    return it;
  };

  int tile = 0, cnt = 0;
  int it = advance(beg, tile, cnt);
  bf16x8 qf[D / 16];
  f32x16 acc_o[D / 32];
  float m_run = -INFINITY, l_run = 0.f;
  auto start_tile = [&](int tl) {
    const int hh = tl / nb, ii = tl - hh * nb;
    const int qr = ii * BLK + wave * 32 + col;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qr < n) w = *reinterpret_cast<const u32x4*>(Q + ((size_t)hh * n + qr) * D + 16 * kk + 8 * g);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[dt][e] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  };
  int jj = 0;
  int j = 0;
  if (it < end) {
    start_tile(tile);
    j = block_of(tile, 0);
    dma_k(tile / nb, j);
  }
  while (it < end) {
    const int h = tile / nb;
    const int i = tile - h * nb;
    // the (tile, block) pair after this one
    int tile2 = tile, cnt2 = cnt, jj2 = jj + 1, it2 = it;
    if (jj2 >= cnt) {
      it2 = advance(it + 1, tile2, cnt2);
      jj2 = 0;
    }
    const bool more = it2 < end;
    const int jn = more ? block_of(tile2, jj2) : j;      // last: harmless reload

    wait_vmcnt<0>();
    lds_barrier();                                     // A
    dma_v(h, j);

    // S^T = K Q^T; the key tiles kt are independent accumulators, so they are
    // interleaved (kk outer) to keep dependent MFMAs apart
    f32x16 s[BLK / 32];
#pragma unroll
    for (int kt = 0; kt < BLK / 32; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kt = 0; kt < BLK / 32; ++kt) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(Ks + k_off<D>(32 * kt + col, 2 * kk + g));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                        qf[kk], s[kt], 0, 0, 0);
      }
    }
    lds_barrier();                                     // B
    dma_k(more ? tile2 / nb : h, jn);

    const int r0 = j * BLK;
    if (r0 + BLK > n) {
      keep_branch();
#pragma unroll
      for (int kt = 0; kt < BLK / 32; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = r0 + 32 * kt + 8 * (e >> 2) + 4 * g + (e & 3);
          if (key >= n) s[kt][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < BLK / 32; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mxs = mx * sl2;
    const bool grow = mxs > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      keep_branch();
      const float m_new = grow ? mxs : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[dt][e] *= alpha;
    }
    const float m_sub = m_run == -INFINITY ? 0.f : m_run;
    // P in bf16; the row sum adds the same rounded values the P.V product uses
    // (v_dot2 with (1, 1): two per instruction)
    uint32_t pk[BLK / 32][8];
#pragma unroll
    for (int kt = 0; kt < BLK / 32; ++kt)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][e], sl2, -m_sub));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][e + 1], sl2, -m_sub));
        pk[kt][e >> 1] = pack_bf16x2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[kt][e >> 1]),
                                                kOnesBf16x2, l_run, false);
      }

    wait_vmcnt<KDMA>();                                // V_j landed (K_next may fly)
    lds_barrier();                                     // C
#pragma unroll
    for (int c = 0; c < BLK / 16; ++c) {
      const u32x4 pb = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1],
                        pk[c >> 1][4 * (c & 1) + 2], pk[c >> 1][4 * (c & 1) + 3]};
      const bf16x8 bop = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int dd = 32 * dt + col;
        const u32x4 av = *reinterpret_cast<const u32x4*>(Vs + vt_off<D, BLK>(dd, 2 * c + g));
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                            bop, acc_o[dt], 0, 0, 0);
      }
    }

    if (jj2 == 0) {
      // tile finished: normalise and store, then set up the next one
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const int qrow = i * BLK + wave * 32 + col;
      if (qrow < n) {
        uint16_t* orow = O + ((size_t)h * n + out_row(a, qrow)) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = 32 * dt + 8 * r4 + 4 * g;
            const u32x2 w = {pack_bf16x2(acc_o[dt][4 * r4 + 0] * inv, acc_o[dt][4 * r4 + 1] * inv),
                             pack_bf16x2(acc_o[dt][4 * r4 + 2] * inv, acc_o[dt][4 * r4 + 3] * inv)};
            *reinterpret_cast<u32x2*>(orow + d0) = w;
          }
      }
      if (more) start_tile(tile2);
    }
    tile = tile2;
    cnt = cnt2;
    jj = jj2;
    it = it2;
    j = jn;
  }
  wait_vmcnt<0>();        // no LDS copy may outlive the workgroup
  if (PERSIST && a.timing) {
    __syncthreads();
    if (tid == 0) stamp_end(a.timing, blockIdx.x, t0);
  }
#endif
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel for tiles of G consecutive q-blocks (group = G = 2 or 3),
// V as tiles.
//
// Every kept (q-block, key block) pair streams a 64 KB K + V^T block (d =
// 128) from L2 into LDS, so one workgroup of G*BLK/32 wavefronts serves G
// consecutive q-blocks of a head and loads each key block once for all of
// them: it walks the union of the G ascending kept lists, and the
// wavefronts of each q-block compute only on the blocks their q-block kept
// (BLK/32 wavefronts of 32 queries per q-block; wavefront w runs on SIMD
// w % 4, so each SIMD holds one wavefront of every q-block).  K and V^T are double
// buffered in four LDS arrays (the loop body is instantiated for both buffer
// assignments, so the compiler sees distinct objects and does not wait on the
// in-flight copy): the copy of union block u+1 is issued after the one barrier
// of block u (by the wavefronts that compute on block u after their score
// product, by the others at once) and overlaps block u's work.  HK is the key
// width of one online-softmax step (the block is processed in BLK/HK steps).
// ---------------------------------------------------------------------------
// The persistent launch (worker lists) and the head-major grid launch (one
// workgroup per tile, worker_offsets == null) run this one compiled body, so
// both give the same bits for a tile.
template <int D, int BLK, int G, int HK, bool CONFINED = false>
__global__ __launch_bounds__(2 * G * BLK) void attn_mfma_tile_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const bool PERSIST = a.worker_offsets != nullptr;
  constexpr int WPQ = BLK / 32;               // wavefronts per q-block
  constexpr int NW = G * WPQ;                 // wavefronts, all q-blocks
  constexpr int CPRK = D / 8;
  constexpr int CPRV = BLK / 8;
  // 1 KB DMA instructions per block (64 lanes x 16 bytes) and the most any
  // wavefront issues: wavefront w takes instructions w, w + NW, ...
  constexpr int NIK = BLK * CPRK / 64;
  constexpr int NIV = D * CPRV / 64;
  constexpr int KDMA = (NIK + NW - 1) / NW;
  constexpr int VDMA = (NIV + NW - 1) / NW;
  static_assert(G >= 2 && G <= 3 && BLK % HK == 0 && HK % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(1024))) uint8_t K0[BLK * D * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t K1[BLK * D * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t V0[D * BLK * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t V1[D * BLK * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp = wave / WPQ;                 // which q-block of the tile
  const int wq = wave % WPQ;                  // 32-query slice inside it
  const int col = lane & 31;
  const int g = lane >> 5;
  const int n = a.n, nb = a.nb, tph = a.tiles_per_head;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  uint16_t* O = static_cast<uint16_t*>(a.o);
  const float sl2 = a.scale_log2;
  // one descriptor per head (head_rsrc): K rows past the end of a head read
  // as zero and the score mask removes them
  const uint32_t kbytes = (uint32_t)((size_t)n * D * 2);
  const uint32_t vbytes = (uint32_t)((size_t)nb * D * BLK * 2);

  // DMA instruction x of this wave fills LDS chunks P = (x*NW + wave)*64 + lane
  // (when x*NW + wave is below the instruction count); consecutive x advance
  // by NW*64 chunks = a whole number of rows that is a multiple of the
  // swizzle period, so the source offset is affine in x
  static_assert((NW * 64 / CPRK) % CPRK == 0 && (NW * 64 / CPRV) % 16 == 0, "swizzle period");
  constexpr uint32_t kStepK = (NW * 64 / CPRK) * D * 2;     // bytes per DMA step, K
  constexpr uint32_t kStepV = (NW * 64 / CPRV) * BLK * 2;   // and V^T
  uint32_t koff, voff;
  {
    const int P = wave * 64 + lane;
    const int r = P / CPRK, pc = P % CPRK;
    koff = (uint32_t)(r * D * 2 + (pc ^ (r & (CPRK - 1))) * 16);
    const int dd = P / CPRV, pv = P % CPRV;
    voff = (uint32_t)(dd * BLK * 2 + (pv ^ vt_swz<BLK>(dd)) * 16);
  }
  auto dma = [&](uint8_t* kb, uint8_t* vb, int h, int j) {
    const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k, h, kbytes);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v, h, vbytes);
    const uint32_t kbase = (uint32_t)j * (BLK * D * 2) + koff;
    const uint32_t vbase = (uint32_t)j * (D * BLK * 2) + voff;
#pragma unroll
    for (int x = 0; x < KDMA; ++x)
      if (NIK % NW == 0 || x * NW + wave < NIK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            krs, (lds_void*)(kb + (x * NW + wave) * 1024), 16, kbase + x * kStepK, 0, 0, 0);
#pragma unroll
    for (int x = 0; x < VDMA; ++x)
      if (NIV % NW == 0 || x * NW + wave < NIV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vrs, (lds_void*)(vb + (x * NW + wave) * 1024), 16, vbase + x * kStepV, 0, 0, 0);
  };

  uint64_t t0 = 0;
  if (PERSIST && a.timing && tid == 0) stamp_start(t0);
  int beg = blockIdx.x, end = blockIdx.x + 1;
  // run-time balancing: the tiles come from claims instead of this
  // workgroup's list alone (see claim below); `end` is then only a sentinel
  const bool dyn = PERSIST && a.claims != nullptr;
  if (PERSIST) {
    beg = ld_uniform(a.worker_offsets + blockIdx.x);
    end = ld_uniform(a.worker_offsets + blockIdx.x + 1);
  }
  if (dyn) end = 0x7fffffff;

  // walk state (wave-uniform): position in the worker list (a position in
  // worker_tiles), the tile's head and first q-block, the G list lengths and
  // cursors, the current union block and which lists hold it (bit g), and
  // the tile's ordinal in this workgroup's sequence
  struct Walk {
    int it, h, i0, c[G], p[G], u, ord, in;
  };
  auto list_at = [&](int h, int i, int p) {
    return min(max(ld_uniform(a.kv_index + ((size_t)h * nb + i) * nb + p), 0), nb - 1);
  };
  auto set_block = [&](Walk& w) {
    int jg[G];
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2)
      jg[g2] = w.p[g2] < w.c[g2] ? list_at(w.h, w.i0 + g2, w.p[g2]) : nb;
    w.u = jg[0];
#pragma unroll
    for (int g2 = 1; g2 < G; ++g2) w.u = min(w.u, jg[g2]);
    w.in = 0;
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2) w.in |= (jg[g2] == w.u) << g2;
  };
  // kept count of q-block i0 + g2 of head h, clamped to [0, nb] (0 past the
  // last q-block): a negative entry must not make the tile look empty
  auto count_at = [&](int h, int i0, int g2) {
    return i0 + g2 < nb ? min(max(ld_uniform(a.kv_count + (size_t)h * nb + i0 + g2), 0), nb) : 0;
  };
  auto zero_rows = [&](int h, int i) {
    const int qr = i * BLK + wq * 32 + col;
    if (i < nb && qr < n) {
      uint16_t* orow = O + ((size_t)h * n + out_row(a, qr)) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * r4 + 4 * g) = u32x2{0u, 0u};
    }
  };
  // Run-time balancing.  Counter claims[w] counts the tiles of worker w's
  // LPT list handed out so far.  A workgroup takes the next tile of its own
  // list while there is one, then the next tile of the list with the most
  // tiles left (with claim_groups = x > 1, only among the lists of its own
  // group, w % x, so the groups stay independent like ranks); every hand-out
  // is one atomic add, so each tile runs exactly once whichever workgroup
  // runs it.  Wave 0 makes the claims and posts the list positions in an LDS
  // ring of four slots; pairs with no kept block are written as zeros by
  // wave 0 while claiming.
  //
  // Ring order.  Tile ordinal k is opened (its slot read, by every wave)
  // before the barrier of the step that runs the last union block of tile
  // k-1.  Slots 0-2 are written before the start-up barrier; the slot of
  // tile k+2 is written by wave 0 after the barrier of the step t that opens
  // tile k.  Tile k+1 takes at least step t+1, so tile k+2 is opened at step
  // t+2 or later, after barrier t+1, which wave 0 reaches only after its
  // write: the read sees it even when every tile has a single union block.
  // The slot's previous value (tile k-2) was read at a step no later than
  // t-2, before that step's barrier, so the write cannot overtake the read.
  __shared__ int mbox[4];
  bool own_done = false;
  const int end_own = PERSIST ? ld_uniform(a.worker_offsets + blockIdx.x + 1) : end;
  auto claim = [&]() -> int {
    const int W = a.n_workers;
    const int own = blockIdx.x;
    while (true) {
      int pos = -1;
      if (!own_done) {
        int j = 0;
        if (lane == 0) j = atomicAdd(a.claims + own, 1);
        j = __builtin_amdgcn_readfirstlane(j);
        if (j < end_own - beg) pos = beg + j;
        else own_done = true;
      }
      if (pos < 0) {
        // the list with the most unclaimed tiles (ties: lowest index)
        int best_rem = 0, best_v = -1;
        // candidates: every list, or (the CONFINED instance, claim_groups =
        // x > 1) the lists of this group only, v = own % x + x * k; a
        // separate instance keeps the group arithmetic out of the default
        // kernel's registers
        int gx = 1, g0 = 0, span = W;
        if constexpr (CONFINED) {
          gx = a.claim_groups;
          g0 = own % gx;
          span = (W - g0 + gx - 1) / gx;
        }
        for (int base = 0; base < span; base += 64) {
          const int v = g0 + gx * (base + lane);
          int rem = 0;
          if (base + lane < span && v != own) {
            const int lo = a.worker_offsets[v], hi = a.worker_offsets[v + 1];
            rem = hi - lo - __hip_atomic_load(a.claims + v, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
          }
          int bv = rem > 0 ? v : -1;
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1) {
            const int orem = __shfl_xor(rem, m, 64);
            const int ov = __shfl_xor(bv, m, 64);
            if (orem > rem || (orem == rem && ov >= 0 && (bv < 0 || ov < bv))) {
              rem = orem;
              bv = ov;
            }
          }
          if (rem > best_rem) {
            best_rem = rem;
            best_v = bv;
          }
        }
        best_v = __builtin_amdgcn_readfirstlane(best_v);
        if (best_v < 0) return -1;                 // every list is exhausted
        int j = 0;
        if (lane == 0) j = atomicAdd(a.claims + best_v, 1);
        j = __builtin_amdgcn_readfirstlane(j);
        const int lo = ld_uniform(a.worker_offsets + best_v);
        const int hi = ld_uniform(a.worker_offsets + best_v + 1);
        if (j >= hi - lo) continue;                // lost the race for it
        pos = lo + j;
      }
      const int tile = ld_uniform(a.worker_tiles + pos);
      const int h = tile / tph;
      const int i0 = (tile - h * tph) * G;
      int any = 0;
#pragma unroll
      for (int g2 = 0; g2 < G; ++g2) any |= count_at(h, i0, g2);
      if (any > 0) return pos;
      // nothing kept: zero the tile's rows here
      for (int r = lane; r < G * BLK; r += 64) {
        const int qr = i0 * BLK + r;
        if (qr < n) {
          u32x4* orow = reinterpret_cast<u32x4*>(O + ((size_t)h * n + out_row(a, qr)) * D);
#pragma unroll
          for (int c = 0; c < D / 8; ++c) orow[c] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  if (dyn) {
    if (wave == 0) {
      const int c0 = claim();
      const int c1 = claim();
      const int c2 = claim();
      if (lane == 0) {
        mbox[0] = c0;
        mbox[1] = c1;
        mbox[2] = c2;
      }
    }
    lds_barrier();
  }
  int ntile = 0;                                // tiles opened so far
  // open the tile at list position it (static lists), or the next claimed
  // one; skips tiles with nothing kept
  auto open_tile = [&](Walk& w, int it) {
    if (dyn) {
      const int pos = __builtin_amdgcn_readfirstlane(mbox[ntile & 3]);
      w.ord = ntile++;
      if (pos < 0) {
        w.it = end;
        return;
      }
      const int tile = ld_uniform(a.worker_tiles + pos);
      const int h = tile / tph;
      const int i0 = (tile - h * tph) * G;
      w.it = pos; w.h = h; w.i0 = i0;
#pragma unroll
      for (int g2 = 0; g2 < G; ++g2) {
        w.c[g2] = count_at(h, i0, g2);
        w.p[g2] = 0;
      }
      set_block(w);
      return;
    }
    while (it < end) {
      const int tile = PERSIST ? ld_uniform(a.worker_tiles + it) : it;
      const int h = tile / tph;
      const int i0 = (tile - h * tph) * G;
      int any = 0;
#pragma unroll
      for (int g2 = 0; g2 < G; ++g2) {
        w.c[g2] = count_at(h, i0, g2);
        any |= w.c[g2];
      }
      if (any > 0) {
        w.it = it; w.h = h; w.i0 = i0;
#pragma unroll
        for (int g2 = 0; g2 < G; ++g2) w.p[g2] = 0;
        w.ord = 0;
        set_block(w);
        return;
      }
      zero_rows(h, i0 + grp);
      ++it;
    }
    w.it = end;
  };
  auto advance = [&](Walk w) {
    bool done = true;
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2) {
      w.p[g2] += (w.in >> g2) & 1;
      done = done && w.p[g2] >= w.c[g2];
    }
    if (done) open_tile(w, w.it + 1);
    else set_block(w);
    return w;
  };

  bf16x8 qf[D / 16];
  f32x16 acc_o[D / 32];
  float m_run = -INFINITY, l_run = 0.f;
  auto start_tile = [&](const Walk& w) {
    const int i = w.i0 + grp;
    const int qr = i * BLK + wq * 32 + col;
    const bool ok = i < nb && qr < n;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 v4 = {0u, 0u, 0u, 0u};
      if (ok) v4 = *reinterpret_cast<const u32x4*>(Q + ((size_t)w.h * n + qr) * D + 16 * kk + 8 * g);
      qf[kk] = __builtin_bit_cast(bf16x8, v4);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[dt][e] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  };
  auto finish_tile = [&](const Walk& w) {
    const int i = w.i0 + grp;
    const int qr = i * BLK + wq * 32 + col;
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (i < nb && qr < n) {
      uint16_t* orow = O + ((size_t)w.h * n + out_row(a, qr)) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * dt + 8 * r4 + 4 * g;
          const u32x2 o2 = {pack_bf16x2(acc_o[dt][4 * r4 + 0] * inv, acc_o[dt][4 * r4 + 1] * inv),
                            pack_bf16x2(acc_o[dt][4 * r4 + 2] * inv, acc_o[dt][4 * r4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = o2;
        }
    }
  };

  // one union block: compute on (kc, vc), prefetch the next one into (kn, vn)
  Walk cur;
  open_tile(cur, beg);
  auto step = [&](uint8_t* kc, uint8_t* vc, uint8_t* kn, uint8_t* vn) {
    const Walk nxt = advance(cur);
    wait_vmcnt<0>();
    lds_barrier();
    // the next block's copies: wavefronts with nothing to compute this step
    // issue their share now, the others after their first S product, so the
    // copies do not compete with the step's first LDS reads (the buffers
    // they fill were released by the barrier above)
    const bool mine = (cur.in >> grp) & 1;
    if (!mine && nxt.it < end) dma(kn, vn, nxt.h, nxt.u);
    if (dyn && nxt.it != cur.it && nxt.it < end && wave == 0) {
      // this step opened tile nxt.ord: post the tile two after it (ring order)
      const int c = claim();
      if (lane == 0) mbox[(nxt.ord + 2) & 3] = c;
    }
    if (mine) {
      // the block in steps of HK keys: an online-softmax step per HK keys
      // keeps the live score / probability registers small
      constexpr int KT = HK / 32;              // 32-key tiles per step
      const int j = cur.u;
      const int r0 = j * BLK;
#pragma unroll
      for (int half = 0; half < BLK / HK; ++half) {
        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const int row = half * HK + 32 * kt + col;
            const u32x4 w4 = *reinterpret_cast<const u32x4*>(kc + k_off<D>(row, 2 * kk + g));
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w4),
                                                            qf[kk], s[kt], 0, 0, 0);
          }
        }
        if (half == 0) {
          // the first half starts right after the barrier with nothing else
          // to overlap: keep kReadAhead K reads in flight ahead of the MFMAs
          // (the default schedule waits on every second read)
          constexpr int kN = (D / 16) * KT;
          constexpr int kReadAhead = kN > 6 ? 6 : kN - 1;
          __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);   // LDS reads
#pragma unroll
          for (int x = 0; x < kN - kReadAhead; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // one read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, kReadAhead, 0);
        }
        if (half == 0 && nxt.it < end) dma(kn, vn, nxt.h, nxt.u);
        if (r0 + half * HK + HK > n) {
          keep_branch();
          // keys at or past n get -inf; the sign of key - n selects, so the
          // mask needs no per-element condition registers
          const int base = r0 + half * HK + 4 * g - n;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int keep = (base + 32 * kt + 8 * (e >> 2) + (e & 3)) >> 31;  // -1: key < n
              s[kt][e] = __uint_as_float((__float_as_uint(s[kt][e]) & (uint32_t)keep) |
                                         (0xff800000u & ~(uint32_t)keep));
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
        mx = max_with_other_half(mx);
        const float mxs = mx * sl2;
        const bool grow = mxs > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          keep_branch();
          const float m_new = grow ? mxs : m_run;
          const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc_o[dt][e] *= alpha;
        }
        const float m_sub = m_run == -INFINITY ? 0.f : m_run;
        uint32_t pk[KT][8];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][e], sl2, -m_sub));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][e + 1], sl2, -m_sub));
            pk[kt][e >> 1] = pack_bf16x2(p0, p1);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[kt][e >> 1]),
                                                    kOnesBf16x2, l_run, false);
          }
        // chunk c (16 keys) of this half = accumulator registers 8*(c%2).. of tile c/2
#pragma unroll
        for (int c = 0; c < HK / 16; ++c) {
          const u32x4 pb = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1],
                            pk[c >> 1][4 * (c & 1) + 2], pk[c >> 1][4 * (c & 1) + 3]};
          const bf16x8 bop = __builtin_bit_cast(bf16x8, pb);
          const int cb = half * (HK / 16) + c;     // chunk index inside the block
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const int dd = 32 * dt + col;
            const u32x4 av = *reinterpret_cast<const u32x4*>(vc + vt_off<D, BLK>(dd, 2 * cb + g));
            acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                bop, acc_o[dt], 0, 0, 0);
          }
        }
      }
    }
    if (nxt.it != cur.it) {
      finish_tile(cur);
      if (nxt.it < end) start_tile(nxt);
    }
    cur = nxt;
    return cur.it < end;
  };

  if (cur.it < end) {
    start_tile(cur);
    dma(K0, V0, cur.h, cur.u);
    while (step(K0, V0, K1, V1) && step(K1, V1, K0, V0)) {
    }
  }
  wait_vmcnt<0>();
  if (PERSIST && a.timing) {
    __syncthreads();
    if (tid == 0) stamp_end(a.timing, blockIdx.x, t0);
  }
#endif
}

__global__ void claims_reset_kernel(int32_t* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0;
}

// key width of one online-softmax step.  Every step pays a fixed cost (the
// scores' MFMAs drain before the row max, the max exchange, the rescale
// vote), so tiles of two q-blocks take the whole block in one step (231
// VGPRs at d = block = 128, no spills); three q-blocks per tile (three
// wavefronts per SIMD, at most 168 VGPRs each) take 32-key steps.
template <int BLK, int G>
constexpr int tile_hk() { return G == 2 ? BLK : 32; }

template <int D, int BLK, int G>
hipError_t launch_mfma_tile(const AttnArgs& a, hipStream_t s) {
  constexpr int HK = tile_hk<BLK, G>();
  constexpr int threads = 2 * G * BLK;
  if (a.worker_offsets && a.claims) {
    hipLaunchKernelGGL(claims_reset_kernel, dim3((a.n_workers + 255) / 256), dim3(256), 0, s,
                       a.claims, a.n_workers);
  }
  if (a.worker_offsets && a.claims && a.claim_groups > 1) {
    hipLaunchKernelGGL((attn_mfma_tile_kernel<D, BLK, G, HK, true>), dim3(a.n_workers),
                       dim3(threads), 0, s, a);
  } else if (a.worker_offsets) {
    hipLaunchKernelGGL((attn_mfma_tile_kernel<D, BLK, G, HK>), dim3(a.n_workers),
                       dim3(threads), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_mfma_tile_kernel<D, BLK, G, HK>),
                       dim3(a.heads * a.tiles_per_head), dim3(threads), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_mfma_dma(const AttnArgs& a, hipStream_t s) {
  using S = MfmaShape<D, BLK>;
  if (a.worker_offsets) {
    hipLaunchKernelGGL((attn_mfma_dma_kernel<D, BLK, true>), dim3(a.n_workers),
                       dim3(S::kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_mfma_dma_kernel<D, BLK, false>), dim3(a.heads * a.nb),
                       dim3(S::kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t s) {
  using S = MfmaShape<D, BLK>;
  if (a.worker_offsets) {
    hipLaunchKernelGGL((attn_mfma_kernel<D, BLK, true>), dim3(a.n_workers),
                       dim3(S::kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_mfma_kernel<D, BLK, false>), dim3(a.heads * a.tiles_per_head),
                       dim3(S::kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int DMAX>
hipError_t launch_simple(const AttnArgs& a, hipStream_t s) {
  if (a.worker_offsets) {
    hipLaunchKernelGGL((attn_simple_kernel<T, DMAX, true>), dim3(a.n_workers),
                       dim3(kSimpleThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_simple_kernel<T, DMAX, false>), dim3(a.heads * a.tiles_per_head),
                       dim3(kSimpleThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_simple_any(const AttnArgs& a, hipStream_t s) {
  if (a.d <= 32) return launch_simple<T, 32>(a, s);
  if (a.d <= 64) return launch_simple<T, 64>(a, s);
  return launch_simple<T, 128>(a, s);
}

}  // namespace

template <typename K>
hipError_t occupancy_of(K kernel, int threads, int* per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, reinterpret_cast<const void*>(kernel),
                                                      threads, 0);
}

hipError_t attn_occupancy(bool bf16, int d, int block, bool v_tiles, int group,
                          int* per_cu) {
  if (attn_has_mfma_instance(bf16, d, block)) {
    const int threads = 2 * block;
#define FV_OCC(D, B)                                                                          \
  if (d == D && block == B) {                                                                 \
    if (v_tiles && group == 2)                                                                \
      return occupancy_of(attn_mfma_tile_kernel<D, B, 2, tile_hk<B, 2>()>, 2 * threads, \
                          per_cu);                                                            \
    if constexpr (B == 128)                                                                   \
      if (v_tiles && group == 3)                                                              \
        return occupancy_of(attn_mfma_tile_kernel<D, B, 3, tile_hk<B, 3>()>,            \
                            3 * threads, per_cu);                                             \
    return v_tiles ? occupancy_of(attn_mfma_dma_kernel<D, B, true>, threads, per_cu)          \
                   : occupancy_of(attn_mfma_kernel<D, B, true>, threads, per_cu);             \
  }
    FV_OCC(128, 128)
    FV_OCC(64, 64)
    FV_OCC(64, 128)
    FV_OCC(128, 64)
#undef FV_OCC
  }
  const int dm = d <= 32 ? 32 : d <= 64 ? 64 : 128;
  if (bf16) {
    if (dm == 32) return occupancy_of(attn_simple_kernel<bf16s, 32, true>, kSimpleThreads, per_cu);
    if (dm == 64) return occupancy_of(attn_simple_kernel<bf16s, 64, true>, kSimpleThreads, per_cu);
    return occupancy_of(attn_simple_kernel<bf16s, 128, true>, kSimpleThreads, per_cu);
  }
  if (dm == 32) return occupancy_of(attn_simple_kernel<float, 32, true>, kSimpleThreads, per_cu);
  if (dm == 64) return occupancy_of(attn_simple_kernel<float, 64, true>, kSimpleThreads, per_cu);
  return occupancy_of(attn_simple_kernel<float, 128, true>, kSimpleThreads, per_cu);
}

bool attn_has_group3_instance(bool bf16, int d, int block, bool v_tiles) {
  return bf16 && v_tiles && block == 128 && (d == 64 || d == 128);
}

bool attn_has_mfma_instance(bool bf16, int d, int block) {
  if (!bf16) return false;
  return (d == 64 || d == 128) && (block == 64 || block == 128);
}

hipError_t launch_sparse_attn(const AttnArgs& a, bool bf16, hipStream_t s) {
  if (attn_has_mfma_instance(bf16, a.d, a.block) && a.v_tiles && a.group == 2) {
    if (a.d == 128 && a.block == 128) return launch_mfma_tile<128, 128, 2>(a, s);
    if (a.d == 64 && a.block == 64) return launch_mfma_tile<64, 64, 2>(a, s);
    if (a.d == 64 && a.block == 128) return launch_mfma_tile<64, 128, 2>(a, s);
    return launch_mfma_tile<128, 64, 2>(a, s);
  }
  if (a.group == 3) {
    // three q-blocks per tile: 128-key blocks with V tiles only (the ABI
    // refuses the rest)
    if (a.d == 128) return launch_mfma_tile<128, 128, 3>(a, s);
    return launch_mfma_tile<64, 128, 3>(a, s);
  }
  if (attn_has_mfma_instance(bf16, a.d, a.block) && a.v_tiles) {
    if (a.d == 128 && a.block == 128) return launch_mfma_dma<128, 128>(a, s);
    if (a.d == 64 && a.block == 64) return launch_mfma_dma<64, 64>(a, s);
    if (a.d == 64 && a.block == 128) return launch_mfma_dma<64, 128>(a, s);
    return launch_mfma_dma<128, 64>(a, s);
  }
  if (attn_has_mfma_instance(bf16, a.d, a.block)) {
    if (a.d == 128 && a.block == 128) return launch_mfma<128, 128>(a, s);
    if (a.d == 64 && a.block == 64) return launch_mfma<64, 64>(a, s);
    if (a.d == 64 && a.block == 128) return launch_mfma<64, 128>(a, s);
    return launch_mfma<128, 64>(a, s);
  }
  if (bf16) return launch_simple_any<bf16s>(a, s);
  return launch_simple_any<float>(a, s);
}

}  // namespace fvattn
