// LPT work list over (head, q-block) tiles for the persistent attention
// kernel.
//
// Source of the problem: after the mask exists every head's load in sparse
// blocks is known, and a few heavy heads set the critical path (aixai.ru
// FVAttn post, "Runtime Load Balancing (RLB)").  On one GPU the balanced
// resource is the set of persistent workgroups; the rule is Graham's LPT:
// tiles in (cost desc, id asc) order, each to the least-loaded worker (lowest
// index on ties).  Exactly one result is correct, and it is reproduced here.
//
// Kernels:
//   lpt_sort_kernel    one 1024-thread workgroup: stable LSD radix sort (4-bit
//                      digits) of tile ids by (max_cost - cost), starting from
//                      the identity order, so ties keep ascending ids.  Each
//                      thread owns a contiguous run of tiles; digit counts are
//                      kept per thread in LDS and scanned in (digit, thread)
//                      order, which makes every pass stable.
//   lpt_assign_kernel  one wavefront: worker loads live in registers (up to 16
//                      per lane, worker w = lane * per + slot, so "lowest
//                      index" = lowest lane, then lowest slot); per tile a
//                      wavefront min-reduction, a ballot for the first holder
//                      and one update.  Loads are kept relative to a running
//                      base so they fit 32 bits.
//   lpt_scatter_kernel writes each tile at worker_offsets[w] + its position in
//                      w's list (assignment order), or
//   lpt_sort_kernel    run again with key = owner, which groups the tiles by
//                      worker with ascending tile ids inside each list (tile
//                      order: the same assignment and loads, executed
//                      head-major inside every worker so that concurrently
//                      running workgroups share K/V blocks in L2).
#include "device_util.h"
#include "internal.h"

// wavefront reduction from the ROCm device library (DPP based)
extern "C" __device__ uint32_t __ockl_wfred_min_u32(uint32_t);

namespace fvattn {
namespace {

constexpr int kSortThreads = 1024;
constexpr int kRadixBits = 4;
constexpr int kRadix = 1 << kRadixBits;

struct SchedWs {
  int32_t* key_a;
  int32_t* id_a;
  int32_t* key_b;
  int32_t* id_b;
  int32_t* owner;   // worker of the k-th tile in LPT order
  int32_t* slot;    // its position in that worker's list
  int32_t* owner_by_tile;  // worker of tile t
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

SchedWs carve(void* ws, int tiles) {
  const size_t one = align_up(sizeof(int32_t) * (size_t)tiles, 256);
  char* b = static_cast<char*>(ws);
  return SchedWs{reinterpret_cast<int32_t*>(b), reinterpret_cast<int32_t*>(b + one),
                 reinterpret_cast<int32_t*>(b + 2 * one),
                 reinterpret_cast<int32_t*>(b + 3 * one),
                 reinterpret_cast<int32_t*>(b + 4 * one),
                 reinterpret_cast<int32_t*>(b + 5 * one),
                 reinterpret_cast<int32_t*>(b + 6 * one)};
}

__device__ inline int clamp_cost(int c) { return min(max(c, 0), kMaxCost); }

// by_owner == false: ids sorted by (cost desc, id asc) -> out (lpt_order)
// by_owner == true:  ids sorted by (owner asc, id asc)  -> out (worker_tiles)
__global__ __launch_bounds__(kSortThreads) void lpt_sort_kernel(
    const int32_t* __restrict__ cost, int tiles, SchedWs ws,
    int32_t* __restrict__ lpt_order, bool by_owner) {
  __shared__ int32_t table[kRadix * kSortThreads];   // [digit][thread], 64 KB
  __shared__ int32_t s_scan[kSortThreads / kWave];
  __shared__ int32_t s_max[kSortThreads / kWave];
  const int tid = threadIdx.x;
  const int per = (tiles + kSortThreads - 1) / kSortThreads;
  const int lo = min(tiles, tid * per), hi = min(tiles, lo + per);

  const int32_t* src = by_owner ? ws.owner_by_tile : cost;
  int mx = 0;
  for (int t = lo; t < hi; ++t) mx = max(mx, clamp_cost(src[t]));
  mx = block_reduce<kSortThreads>(mx, s_max, [](int a, int b) { return max(a, b); });
  int bits = 0;
  while ((1 << bits) <= mx) ++bits;
  const int passes = (bits + kRadixBits - 1) / kRadixBits;

  // pass input: identity order with key = max - cost
  int32_t* kin = ws.key_a;
  int32_t* iin = ws.id_a;
  int32_t* kout = ws.key_b;
  int32_t* iout = ws.id_b;
  for (int t = lo; t < hi; ++t) {
    const int c = clamp_cost(src[t]);
    kin[t] = by_owner ? c : mx - c;
    iin[t] = t;
  }
  if (passes == 0) {
    // every key is zero: identity order
    for (int t = lo; t < hi; ++t) lpt_order[t] = t;
    return;
  }
  __syncthreads();
  __threadfence_block();

  for (int ps = 0; ps < passes; ++ps) {
    const int sh = ps * kRadixBits;
    const bool last = ps == passes - 1;
#pragma unroll
    for (int dg = 0; dg < kRadix; ++dg) table[dg * kSortThreads + tid] = 0;
    for (int t = lo; t < hi; ++t) table[((kin[t] >> sh) & (kRadix - 1)) * kSortThreads + tid] += 1;
    __syncthreads();
    // exclusive scan of the whole table in (digit, thread) order: thread u
    // owns entries [u*16, u*16+16).
    int run = 0;
    int local[kRadix];
#pragma unroll
    for (int e = 0; e < kRadix; ++e) {
      local[e] = run;
      run += table[tid * kRadix + e];
    }
    int total;
    const int base = block_exclusive_scan<kSortThreads>(run, s_scan, total);
#pragma unroll
    for (int e = 0; e < kRadix; ++e) table[tid * kRadix + e] = base + local[e];
    __syncthreads();
    for (int t = lo; t < hi; ++t) {
      const int key = kin[t];
      const int slot = table[((key >> sh) & (kRadix - 1)) * kSortThreads + tid]++;
      if (last) {
        lpt_order[slot] = iin[t];
      } else {
        kout[slot] = key;
        iout[slot] = iin[t];
      }
    }
    // make this pass's global writes visible to the whole workgroup
    __threadfence_block();
    __syncthreads();
    int32_t* tk = kin; kin = kout; kout = tk;
    int32_t* ti = iin; iin = iout; iout = ti;
  }
}

template <int PER>
__global__ __launch_bounds__(kWave) void lpt_assign_kernel(
    const int32_t* __restrict__ cost, const int32_t* __restrict__ lpt_order,
    int tiles, int n_workers, SchedWs ws, int32_t* __restrict__ worker_offsets,
    int64_t* __restrict__ worker_load) {
  const int lane = threadIdx.x;
  uint32_t rel[PER];      // load - base
  int32_t cnt[PER];
  constexpr uint32_t kInvalid = 0xffffffffu;
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    rel[s] = (lane * PER + s < n_workers) ? 0u : kInvalid;
    cnt[s] = 0;
  }
  uint64_t base = 0;
  uint32_t lmin = kInvalid;
#pragma unroll
  for (int s = 0; s < PER; ++s) lmin = min(lmin, rel[s]);

  for (int k0 = 0; k0 < tiles; k0 += kWave) {
    const int kk = k0 + lane;
    int my_tile = 0, my_cost = 0;
    if (kk < tiles) {
      my_tile = lpt_order[kk];
      my_cost = clamp_cost(cost[my_tile]);
    }
    int my_owner = 0, my_slot = 0;
    const int nstep = min(kWave, tiles - k0);
    for (int j = 0; j < nstep; ++j) {
      // broadcast the j-th tile's cost, find the least-loaded worker
      const uint32_t c = (uint32_t)__builtin_amdgcn_readlane(my_cost, j);
      const uint32_t gmin = __ockl_wfred_min_u32(lmin);
      const uint64_t hit = __ballot(lmin == gmin);
      const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
      int w = 0, pos = 0;
      if (lane == L) {
        bool done = false;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
          if (!done && rel[s] == gmin) {
            done = true;
            w = lane * PER + s;
            pos = cnt[s];
            rel[s] += c;
            cnt[s] += 1;
          }
        }
        lmin = kInvalid;
#pragma unroll
        for (int s = 0; s < PER; ++s) lmin = min(lmin, rel[s]);
      }
      w = __builtin_amdgcn_readlane(w, L);
      pos = __builtin_amdgcn_readlane(pos, L);
      if (lane == j) {
        my_owner = w;
        my_slot = pos;
      }
      // keep relative loads small: rebase when the minimum grows large
      if (gmin > (1u << 30)) {
        base += gmin;
#pragma unroll
        for (int s = 0; s < PER; ++s)
          if (rel[s] != kInvalid) rel[s] -= gmin;
        lmin = kInvalid;
#pragma unroll
        for (int s = 0; s < PER; ++s) lmin = min(lmin, rel[s]);
      }
    }
    if (kk < tiles) {
      ws.owner[kk] = my_owner;
      ws.slot[kk] = my_slot;
      ws.owner_by_tile[my_tile] = my_owner;
    }
  }
  // loads and list offsets
  int my_total = 0;
#pragma unroll
  for (int s = 0; s < PER; ++s) my_total += cnt[s];
  const int incl = wave_inclusive_scan(my_total);
  int off = incl - my_total;
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    const int w = lane * PER + s;
    if (w < n_workers) {
      worker_offsets[w] = off;
      worker_load[w] = (int64_t)(base + rel[s]);
      off += cnt[s];
    }
  }
  if (lane == kWave - 1) worker_offsets[n_workers] = incl;
}

__global__ __launch_bounds__(256) void lpt_scatter_kernel(
    const int32_t* __restrict__ lpt_order, int tiles, SchedWs ws,
    const int32_t* __restrict__ worker_offsets, int32_t* __restrict__ worker_tiles) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < tiles) worker_tiles[worker_offsets[ws.owner[k]] + ws.slot[k]] = lpt_order[k];
}

}  // namespace

size_t schedule_workspace_bytes(int heads, int n_qblocks, int n_workers) {
  (void)n_workers;
  const size_t tiles = (size_t)heads * n_qblocks;
  return 7 * align_up(sizeof(int32_t) * tiles, 256);
}

hipError_t launch_schedule(const int32_t* kv_count, int tiles, int n_workers,
                           bool tile_order, int32_t* lpt_order, int32_t* worker_offsets,
                           int32_t* worker_tiles, int64_t* worker_load, void* wsp,
                           hipStream_t s) {
  SchedWs ws = carve(wsp, tiles);
  hipLaunchKernelGGL(lpt_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, kv_count,
                     tiles, ws, lpt_order, false);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per = (n_workers + kWave - 1) / kWave;
#define FV_ASSIGN(P)                                                                 \
  hipLaunchKernelGGL(lpt_assign_kernel<P>, dim3(1), dim3(kWave), 0, s, kv_count,      \
                     lpt_order, tiles, n_workers, ws, worker_offsets, worker_load)
  if (per <= 1) FV_ASSIGN(1);
  else if (per <= 2) FV_ASSIGN(2);
  else if (per <= 4) FV_ASSIGN(4);
  else if (per <= 8) FV_ASSIGN(8);
  else FV_ASSIGN(16);
#undef FV_ASSIGN
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tile_order) {
    hipLaunchKernelGGL(lpt_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, kv_count,
                       tiles, ws, worker_tiles, true);
  } else {
    hipLaunchKernelGGL(lpt_scatter_kernel, dim3((tiles + 255) / 256), dim3(256), 0, s,
                       lpt_order, tiles, ws, worker_offsets, worker_tiles);
  }
  return hipGetLastError();
}

}  // namespace fvattn
