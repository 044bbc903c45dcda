// LPT work list over (head, q-block) tiles for the persistent attention
// kernel.
//
// A tile is `group` consecutive q-blocks of one head (1 or 2; the attention
// kernel that shares K/V tiles between two q-blocks works on pairs); its cost
// is the sum of their kept-block counts.
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
//   lpt_assign_kernel  one 1024-thread workgroup, exact greedy in batches:
//                      workers sorted by (load, index) in LDS; a run of tiles
//                      goes to the sorted workers in order for as long as each
//                      is still the greedy minimum (prefix-minimum test), then
//                      the keys are re-sorted.  Near-equal costs give batches
//                      of about one tile per worker.
//   lpt_scatter_kernel writes each tile at worker_offsets[w] + its position in
//                      w's list (assignment order), or
//   lpt_sort_kernel    run again with key = owner, which groups the tiles by
//                      worker with ascending tile ids inside each list (tile
//                      order: the same assignment and loads, executed
//                      head-major inside every worker so that concurrently
//                      running workgroups share K/V blocks in L2).
#include "device_util.h"
#include "internal.h"

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
  int32_t* group_cost;     // per-tile cost when a tile spans several q-blocks
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
                 reinterpret_cast<int32_t*>(b + 6 * one),
                 reinterpret_cast<int32_t*>(b + 7 * one)};
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

// Batched exact LPT.  Workers are kept sorted by key = load * 2048 + w in LDS
// (so "smallest key" = least load, lowest index on ties).  For the next tiles
// of the LPT order, tile k+s is tentatively given to the worker at sorted
// position s; the greedy rule would make the same choice exactly when that
// worker's key is below every key already raised in this batch, i.e. below
// the prefix minimum of (key + cost << 11) over positions < s.  The batch is
// cut at the first position where this fails, the raised keys are written
// back and the array is re-sorted (bitonic).  Zero-cost tiles do not change
// any load: they all go to the current minimum.
constexpr int kAssignThreads = 1024;
constexpr int kMaxWorkersPow2 = 2048;
constexpr int kWorkerBits = 11;

__global__ __launch_bounds__(kAssignThreads) void lpt_assign_kernel(
    const int32_t* __restrict__ cost, const int32_t* __restrict__ lpt_order,
    int tiles, int n_workers, SchedWs ws, int32_t* __restrict__ worker_offsets,
    int64_t* __restrict__ worker_load) {
  __shared__ uint64_t key[kMaxWorkersPow2];
  __shared__ uint64_t tmp[kMaxWorkersPow2];
  __shared__ int32_t cnt[kMaxWorkersPow2];
  __shared__ int32_t s_red[kAssignThreads / kWave];
  __shared__ int32_t s_scan[kAssignThreads / kWave];
  const int tid = threadIdx.x;
  int wp = 1;
  while (wp < n_workers) wp <<= 1;
  constexpr uint64_t kInf = ~0ull;
  for (int x = tid; x < wp; x += kAssignThreads) {
    key[x] = x < n_workers ? (uint64_t)x : kInf;
    cnt[x] = 0;
  }
  __syncthreads();

  auto sort_keys = [&]() {
    for (int kk = 2; kk <= wp; kk <<= 1) {
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int x = tid; x < wp; x += kAssignThreads) {
          const int y = x ^ jj;
          if (y > x) {
            const uint64_t a = key[x], b = key[y];
            const bool up = (x & kk) == 0;
            if (up ? (a > b) : (a < b)) {
              key[x] = b;
              key[y] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  };

  int k = 0;
  while (k < tiles) {
    const int bmax = min(n_workers, tiles - k);
    // raised keys, and zero-cost detection
    int zero_at = bmax;
    for (int x = tid; x < wp; x += kAssignThreads) {
      uint64_t nk = kInf;
      if (x < bmax) {
        const uint32_t c = (uint32_t)clamp_cost(cost[lpt_order[k + x]]);
        nk = key[x] + ((uint64_t)c << kWorkerBits);
        if (c == 0) zero_at = min(zero_at, x);
      }
      tmp[x] = nk;
    }
    zero_at = block_reduce<kAssignThreads>(zero_at, s_red, [](int a, int b) { return min(a, b); });
    if (zero_at == 0) {
      // the rest of the order costs nothing: every remaining tile goes to
      // the least-loaded worker, keeping its list order
      const int w0 = (int)(key[0] & ((1u << kWorkerBits) - 1));
      const int base = cnt[w0];
      for (int t = k + tid; t < tiles; t += kAssignThreads) {
        ws.owner[t] = w0;
        ws.slot[t] = base + (t - k);
      }
      __syncthreads();
      if (tid == 0) cnt[w0] = base + (tiles - k);
      __syncthreads();
      break;
    }
    // exclusive prefix minimum of tmp over positions (Hillis-Steele in LDS)
    __syncthreads();
    for (int off = 1; off < wp; off <<= 1) {
      uint64_t v[kMaxWorkersPow2 / kAssignThreads];
      int e = 0;
      for (int x = tid; x < wp; x += kAssignThreads, ++e)
        v[e] = x >= off ? min(tmp[x], tmp[x - off]) : tmp[x];
      __syncthreads();
      e = 0;
      for (int x = tid; x < wp; x += kAssignThreads, ++e) tmp[x] = v[e];
      __syncthreads();
    }
    // tmp[x] is now the inclusive prefix minimum; position s is accepted when
    // key[s] < prefix_min(s - 1)
    int cut = min(bmax, zero_at);
    for (int x = tid; x < cut; x += kAssignThreads)
      if (x > 0 && key[x] >= tmp[x - 1]) cut = min(cut, x);
    cut = block_reduce<kAssignThreads>(cut, s_red, [](int a, int b) { return min(a, b); });
    // assign, raise keys (each worker appears once in a batch)
    for (int x = tid; x < cut; x += kAssignThreads) {
      const uint64_t kx = key[x];
      const int w = (int)(kx & ((1u << kWorkerBits) - 1));
      const uint32_t c = (uint32_t)clamp_cost(cost[lpt_order[k + x]]);
      ws.owner[k + x] = w;
      ws.slot[k + x] = cnt[w];
      cnt[w] += 1;
      key[x] = kx + ((uint64_t)c << kWorkerBits);
    }
    __syncthreads();
    sort_keys();
    k += cut;
  }

  // owner by tile, list offsets and loads
  for (int t = tid; t < tiles; t += kAssignThreads) ws.owner_by_tile[lpt_order[t]] = ws.owner[t];
  // exclusive scan of cnt over workers: contiguous chunk per thread
  const int per = (n_workers + kAssignThreads - 1) / kAssignThreads;
  const int lo = min(n_workers, tid * per), hi = min(n_workers, lo + per);
  int run = 0;
  for (int w = lo; w < hi; ++w) run += cnt[w];
  int total;
  int off = block_exclusive_scan<kAssignThreads>(run, s_scan, total);
  for (int w = lo; w < hi; ++w) {
    worker_offsets[w] = off;
    off += cnt[w];
  }
  if (tid == 0) worker_offsets[n_workers] = total;
  for (int x = tid; x < n_workers; x += kAssignThreads) {
    const uint64_t kx = key[x];
    worker_load[kx & ((1u << kWorkerBits) - 1)] = (int64_t)(kx >> kWorkerBits);
  }
}

// cost of tile t = (h, m) covering q-blocks [m*group, min(nq, (m+1)*group))
__global__ __launch_bounds__(256) void group_cost_kernel(
    const int32_t* __restrict__ kv_count, int nq, int group, int tiles_per_head,
    int tiles, int32_t* __restrict__ out) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= tiles) return;
  const int h = t / tiles_per_head, m = t - h * tiles_per_head;
  int c = 0;
  for (int i = m * group; i < min(nq, (m + 1) * group); ++i)
    c += min(max(kv_count[(size_t)h * nq + i], 0), kMaxCost);
  out[t] = min(c, kMaxCost);
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
  return 8 * align_up(sizeof(int32_t) * tiles, 256);
}

hipError_t launch_schedule(const int32_t* kv_count, int heads, int n_qblocks, int group,
                           int n_workers, bool tile_order, int32_t* lpt_order,
                           int32_t* worker_offsets, int32_t* worker_tiles,
                           int64_t* worker_load, void* wsp, hipStream_t s) {
  const int per_head = (n_qblocks + group - 1) / group;
  const int tiles = heads * per_head;
  SchedWs ws = carve(wsp, heads * n_qblocks);
  const int32_t* cost = kv_count;
  if (group > 1) {
    hipLaunchKernelGGL(group_cost_kernel, dim3((tiles + 255) / 256), dim3(256), 0, s,
                       kv_count, n_qblocks, group, per_head, tiles, ws.group_cost);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    cost = ws.group_cost;
  }
  hipLaunchKernelGGL(lpt_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, cost,
                     tiles, ws, lpt_order, false);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lpt_assign_kernel, dim3(1), dim3(kAssignThreads), 0, s, cost,
                     lpt_order, tiles, n_workers, ws, worker_offsets, worker_load);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tile_order) {
    hipLaunchKernelGGL(lpt_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, cost,
                       tiles, ws, worker_tiles, true);
  } else {
    hipLaunchKernelGGL(lpt_scatter_kernel, dim3((tiles + 255) / 256), dim3(256), 0, s,
                       lpt_order, tiles, ws, worker_offsets, worker_tiles);
  }
  return hipGetLastError();
}

}  // namespace fvattn
