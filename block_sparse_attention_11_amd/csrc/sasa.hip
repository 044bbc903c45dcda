// Slack-aware sparse augmentation (SASA) and the head moves of runtime load
// balancing (RLB), on the XCD worker groups of one GPU.
//
// Sources: after balancing, ranks off the critical path wait for it; SASA
// spends that idle time on extra high-value blocks on those ranks only,
// taken from the blocks the mask skipped, in importance order, within the
// idle-time budget (aixai.ru FVAttn post, section "Slack-Aware Sparse
// Augmentation (SASA)"; PaperDaily FVAttn article, SASA paragraphs).  The
// imbalance factor picks the regime with thresholds k1 = 1.05 and k2 = 1.10
// (nothing, SASA alone, RLB then SASA); n1 = 0.8 and n2 = 0.07 set how much
// is added and when (same section).  RLB moves at most one local head per
// rank, heavy heads from overloaded to underloaded ranks (aixai.ru post,
// section "Runtime Load Balancing (RLB)").
//
// Readings (one GPU): ranks are the G worker groups (worker w in group
// w % G, one XCD each for G = 8); heads start in contiguous groups, head h
// in group h*G/H; loads are kept blocks; rho = max/mean of the group loads.
// RLB: while the critical group (largest load, lowest index) has given no
// head, move its heaviest not-yet-moved head (lowest index on ties) with
// load > 0 and load_t + load_h < load_c to the least-loaded group t; a move
// costs no transfer on one GPU.  A group with slack = max - load >= n2 * max
// gets floor(n1 * slack) extra blocks: its skipped blocks with the largest
// routing importance P[h,i,j], ties by (h, i, j) ascending.  Decisions on
// rho, the trigger and the budget are taken in float64.
//
// Kernels:
//   sasa_plan_kernel      one workgroup: groups, loads, rho, mode, moves,
//                         budgets
//   sasa_rowstats_kernel  one workgroup per routing row: max and sum of the
//                         row softmax with the routing pass's arithmetic, so
//                         P = expf(z - max) / sum has the same bits
//   sasa_hist_kernel      one pass of an 8-bit-digit radix select: histogram
//                         of the keys (bits of P, plus one) of each group's
//                         skipped blocks that match the digits fixed so far
//   sasa_pick_kernel      per group: the next digit of the threshold key
//   sasa_tie_kernel       per group, in (h, i) order: offsets of the blocks
//                         whose key equals the threshold
//   sasa_apply_kernel     one workgroup per row: add the chosen blocks, then
//                         mask row, kv_count and the ascending kv_index list
#include <math.h>

#include "device_util.h"
#include "internal.h"

namespace fvattn {
namespace {

constexpr int kRowThreads = 256;
constexpr int kPlanThreads = 256;

__device__ inline int clamp_group(int g, int G) { return min(max(g, 0), G - 1); }

// ---------------------------------------------------------------------------
// Plan.  Integer loads, float64 decisions; mostly one thread (H <= 4096 and
// G <= 64 keep it to a few hundred thousand steps at worst).
// info: [0] mode, [1] moves, [2, 2+G) group loads before, [2+G, 2+2G) after.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void sasa_plan_kernel(
    const int64_t* __restrict__ head_load, int H, int G, double k1, double k2, double n1,
    double n2, int32_t* __restrict__ head_group, int64_t* __restrict__ budget,
    int64_t* __restrict__ info) {
  __shared__ int32_t grp[kMaxSasaHeads];
  __shared__ uint8_t moved[kMaxSasaHeads];
  __shared__ int64_t loads[kMaxSasaGroups];
  __shared__ uint8_t gave[kMaxSasaGroups];
  const int tid = threadIdx.x;
  for (int h = tid; h < H; h += kPlanThreads) {
    grp[h] = (int32_t)((int64_t)h * G / H);
    moved[h] = 0;
  }
  for (int g = tid; g < G; g += kPlanThreads) gave[g] = 0;
  __syncthreads();
  if (tid != 0) return;
  auto sum_loads = [&]() {
    for (int g = 0; g < G; ++g) loads[g] = 0;
    for (int h = 0; h < H; ++h) loads[grp[h]] += head_load[h];
  };
  sum_loads();
  int64_t total = 0, mx = loads[0];
  for (int g = 0; g < G; ++g) {
    total += loads[g];
    mx = loads[g] > mx ? loads[g] : mx;
    info[2 + g] = loads[g];
  }
  const double rho = total == 0 ? 1.0 : (double)mx * (double)G / (double)total;
  const int mode = rho < k1 ? 0 : (rho < k2 ? 1 : 2);
  int nmoves = 0;
  if (mode == 2) {
    while (true) {
      int c = 0, t = 0;
      for (int g = 1; g < G; ++g) {
        if (loads[g] > loads[c]) c = g;
        if (loads[g] < loads[t]) t = g;
      }
      if (gave[c] || c == t) break;
      int pick = -1;
      for (int h = 0; h < H; ++h) {
        if (grp[h] != c || moved[h] || head_load[h] <= 0) continue;
        if (loads[t] + head_load[h] >= loads[c]) continue;
        if (pick < 0 || head_load[h] > head_load[pick]) pick = h;
      }
      if (pick < 0) break;
      grp[pick] = t;
      moved[pick] = 1;
      gave[c] = 1;
      loads[c] -= head_load[pick];
      loads[t] += head_load[pick];
      ++nmoves;
    }
  }
  int64_t lmax = loads[0];
  for (int g = 1; g < G; ++g) lmax = loads[g] > lmax ? loads[g] : lmax;
  for (int g = 0; g < G; ++g) {
    info[2 + G + g] = loads[g];
    int64_t b = 0;
    if (mode != 0 && lmax > 0) {
      const int64_t slack = lmax - loads[g];
      if ((double)slack >= n2 * (double)lmax) b = (int64_t)floor(n1 * (double)slack);
    }
    budget[g] = b;
  }
  for (int h = 0; h < H; ++h) head_group[h] = grp[h];
  info[0] = mode;
  info[1] = nmoves;
}

// ---------------------------------------------------------------------------
// Augmentation.
// ---------------------------------------------------------------------------
struct GroupSel {
  uint32_t prefix;   // threshold key digits fixed so far
  int32_t all;       // take every skipped block of the group
  int64_t need;      // blocks still to choose at or below the prefix
};

// max and sum of exp(z - max) over a row, in the routing pass's order
__global__ __launch_bounds__(kRowThreads) void sasa_rowstats_kernel(
    const float* __restrict__ z, int nb, float2* __restrict__ stats) {
  __shared__ float s_red[kRowThreads / kWave];
  const size_t row = (size_t)blockIdx.y * nb + blockIdx.x;
  const float* zr = z + row * nb;
  const int tid = threadIdx.x;
  float mx = -INFINITY;
  for (int j = tid; j < nb; j += kRowThreads) mx = fmaxf(mx, zr[j]);
  mx = block_reduce<kRowThreads>(mx, s_red, [](float a, float b) { return fmaxf(a, b); });
  float sum = 0.f;
  for (int j = tid; j < nb; j += kRowThreads) sum += expf(zr[j] - mx);
  sum = block_reduce<kRowThreads>(sum, s_red, [](float a, float b) { return a + b; });
  if (tid == 0) stats[row] = make_float2(mx, sum);
}

// importance key of a skipped block: float bits of P plus one (P >= 0, so
// the order of the keys is the order of P; 0 is never a key)
__device__ inline uint32_t block_key(float zj, float2 st) {
  const float pj = expf(zj - st.x) / st.y;
  return __float_as_uint(pj) + 1u;
}

__global__ void sasa_init_kernel(const int64_t* __restrict__ budget, int G,
                                 GroupSel* __restrict__ sel, uint32_t* __restrict__ hist,
                                 int64_t* __restrict__ added) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < G) {
    sel[t].prefix = 0u;
    sel[t].all = 0;
    sel[t].need = budget[t] > 0 ? budget[t] : 0;
    added[t] = 0;
  }
  if (t < G * 256) hist[t] = 0u;
}

// one radix pass over digit (key >> shift) & 255 of the keys that match the
// digits above it
__global__ __launch_bounds__(kRowThreads) void sasa_hist_kernel(
    const float* __restrict__ z, const float2* __restrict__ stats,
    const uint8_t* __restrict__ mask, const int32_t* __restrict__ head_group, int G, int nb,
    const GroupSel* __restrict__ sel, int shift, uint32_t* __restrict__ hist) {
  __shared__ uint32_t lh[256];
  const int h = blockIdx.y;
  const int g = clamp_group(head_group[h], G);
  const GroupSel s = sel[g];
  if (s.need <= 0 || s.all) return;                // uniform per workgroup
  const int tid = threadIdx.x;
  lh[tid] = 0u;
  __syncthreads();
  const size_t row = (size_t)h * nb + blockIdx.x;
  const float* zr = z + row * nb;
  const uint8_t* mr = mask + row * nb;
  const float2 st = stats[row];
  const uint32_t hi = shift >= 24 ? 0u : ~((1u << (shift + 8)) - 1u);
  for (int j = tid; j < nb; j += kRowThreads) {
    if (mr[j]) continue;
    const uint32_t key = block_key(zr[j], st);
    if ((key & hi) == (s.prefix & hi)) atomicAdd(&lh[(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (lh[tid]) atomicAdd(&hist[g * 256 + tid], lh[tid]);
}

// per group: fix the next digit of the need-th largest key, clear the
// histogram for the next pass
__global__ void sasa_pick_kernel(uint32_t* __restrict__ hist, GroupSel* __restrict__ sel,
                                 int G, int shift) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= G) return;
  uint32_t* hg = hist + g * 256;
  GroupSel s = sel[g];
  if (s.need > 0 && !s.all) {
    if (shift == 24) {
      int64_t total = 0;
      for (int d = 0; d < 256; ++d) total += hg[d];
      if (total <= s.need) {       // the budget covers every skipped block
        s.all = 1;
        s.need = total;
      }
    }
    if (!s.all) {
      int64_t above = 0;
      for (int d = 255; d >= 0; --d) {
        const int64_t c = hg[d];
        if (above + c >= s.need) {
          s.prefix |= (uint32_t)d << shift;
          s.need -= above;
          break;
        }
        above += c;
      }
    }
    sel[g] = s;
  }
  for (int d = 0; d < 256; ++d) hg[d] = 0u;
}

// per row: skipped blocks whose key equals the group's threshold
__global__ __launch_bounds__(kRowThreads) void sasa_tiecount_kernel(
    const float* __restrict__ z, const float2* __restrict__ stats,
    const uint8_t* __restrict__ mask, const int32_t* __restrict__ head_group, int G, int nb,
    const GroupSel* __restrict__ sel, int32_t* __restrict__ rowties) {
  __shared__ int32_t s_red[kRowThreads / kWave];
  const int h = blockIdx.y;
  const size_t row = (size_t)h * nb + blockIdx.x;
  const GroupSel s = sel[clamp_group(head_group[h], G)];
  int cnt = 0;
  if (s.need > 0 && !s.all) {
    const float* zr = z + row * nb;
    const uint8_t* mr = mask + row * nb;
    const float2 st = stats[row];
    for (int j = threadIdx.x; j < nb; j += kRowThreads)
      if (!mr[j] && block_key(zr[j], st) == s.prefix) ++cnt;
  }
  cnt = block_reduce<kRowThreads>(cnt, s_red, [](int a, int b) { return a + b; });
  if (threadIdx.x == 0) rowties[row] = cnt;
}

// one workgroup: tie offsets in (h, i) order within each group
__global__ __launch_bounds__(1024) void sasa_tie_kernel(
    const int32_t* __restrict__ rowties, const int32_t* __restrict__ head_group, int H, int G,
    int nb, int64_t* __restrict__ rowoff) {
  __shared__ int64_t run[kMaxSasaGroups];
  __shared__ int64_t s_scan[1024 / kWave];
  const int tid = threadIdx.x;
  if (tid < G) run[tid] = 0;
  __syncthreads();
  const int per = (nb + 1023) / 1024;
  for (int h = 0; h < H; ++h) {
    const int g = clamp_group(head_group[h], G);
    const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
    int64_t mine = 0;
    for (int i = i0; i < i1; ++i) mine += rowties[(size_t)h * nb + i];
    int64_t tot;
    int64_t pos = block_exclusive_scan<1024>(mine, s_scan, tot);
    const int64_t base = run[g];
    for (int i = i0; i < i1; ++i) {
      rowoff[(size_t)h * nb + i] = base + pos;
      pos += rowties[(size_t)h * nb + i];
    }
    __syncthreads();
    if (tid == 0) run[g] = base + tot;
    __syncthreads();
  }
}

// one workgroup per row of a group with a budget: add the chosen blocks and
// rebuild the row's mask, kv_count and ascending kv_index
__global__ __launch_bounds__(kRowThreads) void sasa_apply_kernel(
    const float* __restrict__ z, const float2* __restrict__ stats, uint8_t* __restrict__ mask,
    const int32_t* __restrict__ head_group, int G, int nb, const int64_t* __restrict__ budget,
    const GroupSel* __restrict__ sel, const int64_t* __restrict__ rowoff,
    int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index,
    int64_t* __restrict__ added) {
  extern __shared__ int32_t flag[];           // [nb]
  __shared__ int32_t s_scan[kRowThreads / kWave];
  const int h = blockIdx.y;
  const int g = clamp_group(head_group[h], G);
  if (budget[g] <= 0) return;                 // uniform per workgroup
  const GroupSel s = sel[g];
  const size_t row = (size_t)h * nb + blockIdx.x;
  const float* zr = z + row * nb;
  uint8_t* mr = mask + row * nb;
  const float2 st = stats[row];
  const int tid = threadIdx.x;
  const int per = (nb + kRowThreads - 1) / kRowThreads;
  const int j0 = min(nb, tid * per), j1 = min(nb, j0 + per);
  // keys equal to the threshold, ranked in j order inside the row
  int mine_ties = 0;
  if (!s.all && s.need > 0)
    for (int j = j0; j < j1; ++j)
      if (!mr[j] && block_key(zr[j], st) == s.prefix) ++mine_ties;
  int total_ties;
  int tie_rank = block_exclusive_scan<kRowThreads>(mine_ties, s_scan, total_ties);
  const int64_t tie_base = (!s.all && s.need > 0) ? rowoff[row] : 0;
  int add = 0;
  for (int j = j0; j < j1; ++j) {
    int f = mr[j];
    if (!f) {
      if (s.all) {
        f = 1;
      } else if (s.need > 0) {
        const uint32_t key = block_key(zr[j], st);
        if (key > s.prefix) {
          f = 1;
        } else if (key == s.prefix) {
          f = tie_base + tie_rank < s.need ? 1 : 0;
          ++tie_rank;
        }
      }
      add += f;
    }
    flag[j] = f;
  }
  __syncthreads();
  int mine = 0;
  for (int j = j0; j < j1; ++j) mine += flag[j];
  int kept;
  int pos = block_exclusive_scan<kRowThreads>(mine, s_scan, kept);
  int32_t* irow = kv_index + row * nb;
  for (int j = j0; j < j1; ++j) {
    mr[j] = (uint8_t)flag[j];
    if (flag[j]) irow[pos++] = j;
  }
  int row_add = block_reduce<kRowThreads>(add, s_scan, [](int a, int b) { return a + b; });
  if (tid == 0) {
    kv_count[row] = kept;
    if (row_add) atomicAdd(reinterpret_cast<unsigned long long*>(added + g),
                           (unsigned long long)row_add);
  }
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct SasaWs {
  float2* stats;
  uint32_t* hist;
  GroupSel* sel;
  int32_t* rowties;
  int64_t* rowoff;
};

SasaWs sasa_carve(void* ws, int heads, int nb, int G) {
  const size_t rows = (size_t)heads * nb;
  char* b = static_cast<char*>(ws);
  SasaWs w;
  size_t off = 0;
  w.stats = reinterpret_cast<float2*>(b + off);
  off += align_up(sizeof(float2) * rows, 256);
  w.hist = reinterpret_cast<uint32_t*>(b + off);
  off += align_up(sizeof(uint32_t) * 256 * (size_t)G, 256);
  w.sel = reinterpret_cast<GroupSel*>(b + off);
  off += align_up(sizeof(GroupSel) * (size_t)G, 256);
  w.rowties = reinterpret_cast<int32_t*>(b + off);
  off += align_up(sizeof(int32_t) * rows, 256);
  w.rowoff = reinterpret_cast<int64_t*>(b + off);
  return w;
}

}  // namespace

size_t sasa_workspace_bytes(int heads, int n, int block, int groups) {
  const size_t nb = ((size_t)n + block - 1) / block;
  const size_t rows = (size_t)heads * nb;
  return align_up(sizeof(float2) * rows, 256) + align_up(sizeof(uint32_t) * 256 * groups, 256) +
         align_up(sizeof(GroupSel) * (size_t)groups, 256) + align_up(sizeof(int32_t) * rows, 256) +
         align_up(sizeof(int64_t) * rows, 256);
}

hipError_t launch_sasa_plan(const int64_t* head_load, int heads, int groups, double k1,
                            double k2, double n1, double n2, int32_t* head_group,
                            int64_t* budget, int64_t* info, hipStream_t s) {
  hipLaunchKernelGGL(sasa_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, head_load, heads,
                     groups, k1, k2, n1, n2, head_group, budget, info);
  return hipGetLastError();
}

hipError_t launch_sasa_augment(const float* z, int heads, int n, int block,
                               const int32_t* head_group, const int64_t* budget, int groups,
                               uint8_t* mask, int32_t* kv_count, int32_t* kv_index,
                               int64_t* head_load, float* head_density, int64_t* added,
                               void* wsp, hipStream_t s) {
  const int nb = (n + block - 1) / block;
  SasaWs ws = sasa_carve(wsp, heads, nb, groups);
  const dim3 rows(nb, heads);
  hipLaunchKernelGGL(sasa_init_kernel, dim3((groups * 256 + 255) / 256), dim3(256), 0, s,
                     budget, groups, ws.sel, ws.hist, added);
  hipLaunchKernelGGL(sasa_rowstats_kernel, rows, dim3(kRowThreads), 0, s, z, nb, ws.stats);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(sasa_hist_kernel, rows, dim3(kRowThreads), 0, s, z, ws.stats, mask,
                       head_group, groups, nb, ws.sel, shift, ws.hist);
    hipLaunchKernelGGL(sasa_pick_kernel, dim3(1), dim3(kMaxSasaGroups), 0, s, ws.hist, ws.sel,
                       groups, shift);
  }
  hipLaunchKernelGGL(sasa_tiecount_kernel, rows, dim3(kRowThreads), 0, s, z, ws.stats, mask,
                     head_group, groups, nb, ws.sel, ws.rowties);
  hipLaunchKernelGGL(sasa_tie_kernel, dim3(1), dim3(1024), 0, s, ws.rowties, head_group, heads,
                     groups, nb, ws.rowoff);
  hipLaunchKernelGGL(sasa_apply_kernel, rows, dim3(kRowThreads), sizeof(int32_t) * nb, s, z,
                     ws.stats, mask, head_group, groups, nb, budget, ws.sel, ws.rowoff, kv_count,
                     kv_index, added);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_head_load(kv_count, heads, nb, head_load, head_density, s);
}

}  // namespace fvattn
