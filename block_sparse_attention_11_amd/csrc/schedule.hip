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
//
// Two-level variant (X > 1 worker groups; worker w is in group w % X, which
// is the XCD a persistent workgroup w runs on when X is the XCD count): the
// pages balance heavy heads between ranks; here heads are spread over the
// groups by the same LPT rule on head loads, and every tile then goes, in the
// global LPT order, to the least-loaded worker of its head's group.  Tiles of
// one head then share one XCD's L2.
//   head_group_kernel      head loads, heads sorted by (load desc, id asc)
//                          in LDS, greedy over the groups in one wavefront
//   group_partition_kernel stable split of the LPT order by group
//   lpt_assign_wave_kernel one wavefront per group of at most 64 workers on
//                          its slice: one lane per worker, the greedy minimum
//                          of key = load << 6 | lane by a DPP reduction per
//                          tile, no LDS and no barrier (a group whose total
//                          cost could overflow the 26-bit load is flagged)
//   lpt_assign_kernel      one workgroup per group on its slice (larger or
//                          flagged groups)
//   worker_offsets_kernel  list offsets from the per-worker counts
#include <mutex>
#include <unordered_map>

#include "device_util.h"
#include "internal.h"

// Scratch of fvattn_schedule_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host the name is only a
// stand-in for the symbol); it takes the device address from
// hipGetSymbolAddress once per device and passes that.
static __device__ __align__(256) unsigned char scratch[fvattn::kNoAllocScratchBytes];

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
  int32_t* head_group;     // two-level: group of every head
  int32_t* gseq;           // two-level: LPT order split by group
  int32_t* wcount;         // two-level: tiles per worker [kMaxWorkers]
  int32_t* goff;           // two-level: start of each group's slice [kMaxGroups + 1]
  int32_t* gslow;          // two-level: 1 = group left to lpt_assign_kernel [kMaxGroups]
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxGroups = 64;
constexpr size_t kSmallSlab = (kMaxWorkers + 2 * kMaxGroups + 1) * sizeof(int32_t);

SchedWs carve(void* ws, int tiles) {
  const size_t one = align_up(sizeof(int32_t) * (size_t)tiles, 256);
  char* b = static_cast<char*>(ws);
  auto at = [&](size_t i) { return reinterpret_cast<int32_t*>(b + i * one); };
  int32_t* small = at(10);
  return SchedWs{at(0), at(1), at(2), at(3), at(4), at(5), at(6), at(7), at(8), at(9),
                 small, small + kMaxWorkers, small + kMaxWorkers + kMaxGroups + 1};
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

// Single level (goff == null): block 0 assigns seq[0 .. tiles) over all
// n_workers workers and also writes the list offsets.  Two-level: block x
// assigns the slice seq[goff[x] .. goff[x+1]) over workers x, x+X, x+2X, ...
// and leaves the offsets to worker_offsets_kernel.  owner/slot are indexed by
// the position in seq.
__global__ __launch_bounds__(kAssignThreads) void lpt_assign_kernel(
    const int32_t* __restrict__ cost, const int32_t* __restrict__ seq_all,
    int tiles_all, int n_workers_all, const int32_t* __restrict__ goff, int n_groups,
    const int32_t* __restrict__ gslow, SchedWs ws, int32_t* __restrict__ worker_offsets,
    int64_t* __restrict__ worker_load) {
  const int grp = blockIdx.x;
  if (gslow && gslow[grp] == 0) return;      // done by lpt_assign_wave_kernel
  const int base_pos = goff ? goff[grp] : 0;
  const int tiles = goff ? goff[grp + 1] - base_pos : tiles_all;
  const int32_t* lpt_order = seq_all + base_pos;
  const int n_workers = goff ? (n_workers_all - grp + n_groups - 1) / n_groups : n_workers_all;
  // local worker j is global worker wg(j)
  auto wg = [&](int j) { return goff ? grp + j * n_groups : j; };
  int32_t* owner = ws.owner + base_pos;
  int32_t* slotp = ws.slot + base_pos;
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
        owner[t] = wg(w0);
        slotp[t] = base + (t - k);
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
      owner[k + x] = wg(w);
      slotp[k + x] = cnt[w];
      cnt[w] += 1;
      key[x] = kx + ((uint64_t)c << kWorkerBits);
    }
    __syncthreads();
    sort_keys();
    k += cut;
  }

  // owner by tile, list offsets and loads
  for (int t = tid; t < tiles; t += kAssignThreads) ws.owner_by_tile[lpt_order[t]] = owner[t];
  if (goff) {
    for (int x = tid; x < n_workers; x += kAssignThreads) {
      const uint64_t kx = key[x];
      const int j = (int)(kx & ((1u << kWorkerBits) - 1));
      worker_load[wg(j)] = (int64_t)(kx >> kWorkerBits);
      ws.wcount[wg(j)] = cnt[j];
    }
    return;
  }
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

// Heads to groups: head loads (sums of their tile costs), heads sorted by
// (load desc, id asc) with a bitonic sort in LDS, then the greedy in wave 0
// (lane x holds group x's load; every head goes to the least-loaded group,
// lowest index on ties).
constexpr int kMaxGroupHeads = 4096;
// a caller's head -> group map, clamped to [0, n_groups)
__global__ void head_group_copy_kernel(const int32_t* __restrict__ in, int heads, int n_groups,
                                       int32_t* __restrict__ out) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h < heads) out[h] = min(max(in[h], 0), n_groups - 1);
}

__global__ __launch_bounds__(1024) void head_group_kernel(
    const int32_t* __restrict__ cost, int heads, int tph, int n_groups,
    int32_t* __restrict__ head_group) {
  __shared__ uint64_t key[kMaxGroupHeads];
  __shared__ uint64_t load[kMaxGroupHeads];
  const int tid = threadIdx.x;
  int hp = 1;
  while (hp < heads) hp <<= 1;
  for (int h = tid; h < hp; h += 1024) {
    uint64_t l = 0;
    if (h < heads)
      for (int m = 0; m < tph; ++m) l += (uint64_t)clamp_cost(cost[(size_t)h * tph + m]);
    load[h] = l;
    // ascending key = (load desc, head asc); loads stay below 2^47
    key[h] = h < heads ? ((((1ull << 47) - 1 - l) << 12) | (uint64_t)h) : ~0ull;
  }
  __syncthreads();
  for (int kk = 2; kk <= hp; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int x = tid; x < hp; x += 1024) {
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
  if (tid < kWave) {
    const int lane = tid;
    uint64_t gl = lane < n_groups ? 0ull : ~0ull;
    for (int r = 0; r < heads; ++r) {
      const int h = (int)(key[r] & 4095u);
      // least-loaded group, lowest index on ties
      uint64_t best = gl;
      int bx = lane;
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) {
        const uint64_t ob = __shfl_xor(best, off, kWave);
        const int ox = __shfl_xor(bx, off, kWave);
        if (ob < best || (ob == best && ox < bx)) {
          best = ob;
          bx = ox;
        }
      }
      if (lane == bx) {
        gl += load[h];
        head_group[h] = bx;
      }
    }
  }
}

// Stable split of the LPT order by the group of each tile's head: seq lists
// the positions of group 0 first, then group 1, ..., each in LPT order;
// goff[x] is where group x starts.  Per-thread counts in LDS, scanned in
// (group, thread) order.
constexpr int kPartThreads = 256;
__global__ __launch_bounds__(kPartThreads) void group_partition_kernel(
    const int32_t* __restrict__ lpt_order, int tiles, int tph,
    const int32_t* __restrict__ head_group, int n_groups, int32_t* __restrict__ seq,
    int32_t* __restrict__ goff) {
  __shared__ int32_t table[kMaxGroups * kPartThreads];   // [group][thread]
  __shared__ int32_t s_scan[kPartThreads / kWave];
  const int tid = threadIdx.x;
  const int per = (tiles + kPartThreads - 1) / kPartThreads;
  const int lo = min(tiles, tid * per), hi = min(tiles, lo + per);
  for (int x = 0; x < kMaxGroups; ++x) table[x * kPartThreads + tid] = 0;
  for (int k = lo; k < hi; ++k) table[head_group[lpt_order[k] / tph] * kPartThreads + tid] += 1;
  __syncthreads();
  // exclusive scan over (group, thread): thread u owns entries [u*64, u*64+64)
  int run = 0;
  int local[kMaxGroups];
#pragma unroll
  for (int e = 0; e < kMaxGroups; ++e) {
    local[e] = run;
    run += table[tid * kMaxGroups + e];
  }
  int total;
  const int base = block_exclusive_scan<kPartThreads>(run, s_scan, total);
#pragma unroll
  for (int e = 0; e < kMaxGroups; ++e) table[tid * kMaxGroups + e] = base + local[e];
  __syncthreads();
  if (tid <= n_groups) goff[tid] = tid < n_groups ? table[tid * kPartThreads] : tiles;
  for (int k = lo; k < hi; ++k) {
    const int t = lpt_order[k];
    seq[table[head_group[t / tph] * kPartThreads + tid]++] = t;
  }
}

// worker_offsets from the per-worker counts of the two-level assignment
__global__ __launch_bounds__(1024) void worker_offsets_kernel(
    const int32_t* __restrict__ wcount, int n_workers, int32_t* __restrict__ worker_offsets) {
  __shared__ int32_t s_scan[1024 / kWave];
  const int tid = threadIdx.x;
  const int per = (n_workers + 1023) / 1024;
  const int lo = min(n_workers, tid * per), hi = min(n_workers, lo + per);
  int run = 0;
  for (int w = lo; w < hi; ++w) run += wcount[w];
  int total;
  int off = block_exclusive_scan<1024>(run, s_scan, total);
  for (int w = lo; w < hi; ++w) {
    worker_offsets[w] = off;
    off += wcount[w];
  }
  if (tid == 0) worker_offsets[n_workers] = total;
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

// Unsigned minimum over the wavefront, returned to every lane: an inclusive
// scan inside each row of 16 lanes (row shifts 1, 2, 4, 8), then the row
// results carried across rows (broadcast of lane 15 to rows 1 and 3, of lane
// 31 to rows 2 and 3), so lane 63 holds the minimum of all 64.  Lanes whose
// DPP source lies outside the row keep the identity 0xffffffff.
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  constexpr int kId = -1;
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x111, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x112, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x114, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x118, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x142, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

constexpr int kLaneBits = 6;                                  // lane index in a key
constexpr int64_t kWaveLoadLimit = (int64_t(1) << (32 - kLaneBits)) - 1;

// The greedy of lpt_assign_kernel for one group of at most 64 workers, one
// tile at a time: worker j of the group is lane j, and the least-loaded
// worker, lowest index on ties, is the minimum of load << 6 | j.  Same
// owners, list positions, counts and loads as lpt_assign_kernel.
__global__ __launch_bounds__(kWave) void lpt_assign_wave_kernel(
    const int32_t* __restrict__ cost, const int32_t* __restrict__ seq_all, int n_workers_all,
    const int32_t* __restrict__ goff, int n_groups, SchedWs ws,
    int64_t* __restrict__ worker_load) {
  const int grp = blockIdx.x;
  const int lane = threadIdx.x;
  const int base_pos = goff[grp];
  const int tiles = goff[grp + 1] - base_pos;
  const int32_t* order = seq_all + base_pos;
  const int nw = (n_workers_all - grp + n_groups - 1) / n_groups;
  // every load stays below the group's total cost
  long long total = 0;
  for (int t = lane; t < tiles; t += kWave) total += clamp_cost(cost[order[t]]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) total += __shfl_xor(total, o);
  if (total >= kWaveLoadLimit) {
    if (lane == 0) ws.gslow[grp] = 1;
    return;
  }
  if (lane == 0) ws.gslow[grp] = 0;
  uint32_t key = lane < nw ? (uint32_t)lane : 0xffffffffu;
  int32_t cnt = 0;
  int32_t* owner = ws.owner + base_pos;
  int32_t* slotp = ws.slot + base_pos;
  for (int k = 0; k < tiles; k += kWave) {
    const int t = k + lane;
    const int32_t mine = t < tiles ? clamp_cost(cost[order[t]]) : 0;
    int32_t my_owner = 0, my_slot = 0;
    const int m = min(kWave, tiles - k);
    for (int i = 0; i < m; ++i) {
      const uint32_t c = (uint32_t)__builtin_amdgcn_readlane(mine, i);
      const uint32_t kmin = wave_min_u32(key);
      const int w = (int)(kmin & (kWave - 1));
      const int32_t s = __builtin_amdgcn_readlane(cnt, w);
      if (lane == w) {
        cnt = s + 1;
        key = kmin + (c << kLaneBits);
      }
      if (lane == i) {
        my_owner = grp + w * n_groups;
        my_slot = s;
      }
    }
    if (t < tiles) {
      owner[t] = my_owner;
      slotp[t] = my_slot;
      ws.owner_by_tile[order[t]] = my_owner;
    }
  }
  if (lane < nw) {
    worker_load[grp + lane * n_groups] = (int64_t)(key >> kLaneBits);
    ws.wcount[grp + lane * n_groups] = cnt;
  }
}

}  // namespace

size_t schedule_workspace_bytes(int heads, int n_qblocks, int n_workers) {
  (void)n_workers;
  const size_t tiles = (size_t)heads * n_qblocks;
  return 10 * align_up(sizeof(int32_t) * tiles, 256) + align_up(kSmallSlab, 256);
}

hipError_t schedule_noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static std::unordered_map<int, void*> by_device;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_device.find(dev);
  if (it == by_device.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = by_device.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

int schedule_max_groups() { return kMaxGroups; }
int schedule_max_group_heads() { return kMaxGroupHeads; }

hipError_t launch_schedule(const int32_t* kv_count, int heads, int n_qblocks, int group,
                           int n_workers, int n_groups, bool tile_order,
                           const int32_t* head_group, int32_t* lpt_order,
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
  const int X = min(n_groups, n_workers);
  const int32_t* seq = lpt_order;
  if (X > 1) {
    if (head_group) {
      hipLaunchKernelGGL(head_group_copy_kernel, dim3((heads + 255) / 256), dim3(256), 0, s,
                         head_group, heads, X, ws.head_group);
    } else {
      hipLaunchKernelGGL(head_group_kernel, dim3(1), dim3(1024), 0, s, cost, heads, per_head, X,
                         ws.head_group);
    }
    hipLaunchKernelGGL(group_partition_kernel, dim3(1), dim3(kPartThreads), 0, s, lpt_order,
                       tiles, per_head, ws.head_group, X, ws.gseq, ws.goff);
    // groups of at most one wavefront of workers take the one-wavefront
    // greedy; lpt_assign_kernel then runs only the groups it flags
    const bool wave = (n_workers + X - 1) / X <= kWave;
    if (wave)
      hipLaunchKernelGGL(lpt_assign_wave_kernel, dim3(X), dim3(kWave), 0, s, cost, ws.gseq,
                         n_workers, ws.goff, X, ws, worker_load);
    hipLaunchKernelGGL(lpt_assign_kernel, dim3(X), dim3(kAssignThreads), 0, s, cost, ws.gseq,
                       tiles, n_workers, ws.goff, X, wave ? ws.gslow : nullptr, ws,
                       worker_offsets, worker_load);
    hipLaunchKernelGGL(worker_offsets_kernel, dim3(1), dim3(1024), 0, s, ws.wcount, n_workers,
                       worker_offsets);
    seq = ws.gseq;
  } else {
    hipLaunchKernelGGL(lpt_assign_kernel, dim3(1), dim3(kAssignThreads), 0, s, cost,
                       lpt_order, tiles, n_workers, (const int32_t*)nullptr, 1,
                       (const int32_t*)nullptr, ws, worker_offsets, worker_load);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tile_order) {
    hipLaunchKernelGGL(lpt_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, cost,
                       tiles, ws, worker_tiles, true);
  } else {
    hipLaunchKernelGGL(lpt_scatter_kernel, dim3((tiles + 255) / 256), dim3(256), 0, s,
                       seq, tiles, ws, worker_offsets, worker_tiles);
  }
  return hipGetLastError();
}

}  // namespace fvattn
