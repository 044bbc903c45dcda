// Internal launch interface between the C ABI (abi.hip) and the kernel files.
// Every launcher only enqueues work on `stream` and returns the HIP status of
// the launch; argument validation has already happened in abi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fvattn {

// bf16 storage element (bit pattern only; arithmetic is done in fp32).
struct bf16s {
  uint16_t bits;
};

// V^T tile layout (fvattn_pack_v): inside each 16-key group of a tile row,
// the four 4-key units are stored in the order 0, 2, 1, 3, so that keys
// {4g..4g+3} and {8+4g..8+4g+3} (the keys one lane of a 32x32x16 MFMA holds
// in the P operand) are 16 contiguous bytes.  Position of key r in its row:
__host__ __device__ inline int vt_pos(int r) {
  const int u = (r >> 2) & 3;
  return (r & ~15) | (((u & 1) << 1 | (u >> 1)) << 2) | (r & 3);
}

// ---- hilbert.hip -----------------------------------------------------------
hipError_t launch_hilbert(int T, int Y, int X, int32_t* perm, int32_t* inv,
                          hipStream_t s);

// ---- permute.hip -----------------------------------------------------------
hipError_t launch_permute_rows(const void* src, void* dst, const int32_t* index,
                               int heads, int n, size_t row_bytes,
                               hipStream_t s);
// bf16 only; requires block % 8 == 0 and d % 8 == 0
hipError_t launch_pack_v(const void* src, void* dst, const int32_t* index, int heads,
                         int n, int d, int block, hipStream_t s);

// ---- route.hip -------------------------------------------------------------
struct RouteWorkspace {
  float* qbar;   // [heads][nB][d]
  float* kbar;   // [heads][nB][d]
  float* z;      // [heads][nB][nB]
};
size_t route_workspace_bytes(int heads, int n, int d, int block);
RouteWorkspace route_carve(void* ws, int heads, int n, int d, int block);
hipError_t launch_route(const void* q, const void* k, bool bf16, int heads,
                        int n, int d, int block, float p, int k_floor,
                        uint8_t* mask, int32_t* kv_count, int32_t* kv_index,
                        int64_t* head_load, float* head_density,
                        const RouteWorkspace& ws, hipStream_t s);
// routing from given pooled means (qbar, kbar [heads][nB][d] fp32); writes
// the scores into ws.z and leaves ws.qbar / ws.kbar alone
hipError_t launch_route_pooled(const float* qbar, const float* kbar, int heads, int n,
                               int d, int block, float p, int k_floor, uint8_t* mask,
                               int32_t* kv_count, int32_t* kv_index, int64_t* head_load,
                               float* head_density, const RouteWorkspace& ws,
                               hipStream_t s);
// dst[h][r] = src[h][index[r]] and pooled[h][j] = the column means of the
// gathered rows of block j, one pass
hipError_t launch_permute_pool(const void* src, void* dst, const int32_t* index, bool bf16,
                               int heads, int n, int d, int block, float* pooled,
                               hipStream_t s);
// per-head sum of kv_count (int64) and density = sum / nB^2
hipError_t launch_head_load(const int32_t* kv_count, int heads, int nb, int64_t* head_load,
                            float* head_density, hipStream_t s);

// ---- schedule.hip ----------------------------------------------------------
constexpr int kMaxWorkers = 2048;
constexpr int kMaxCost = 65535;
size_t schedule_workspace_bytes(int heads, int n_qblocks, int n_workers);
// tiles = heads * ceil(n_qblocks / group); tile t = h * ceil(nq/group) + m
// head_group (nullable, n_groups > 1): the group of every head, used as
// given instead of the LPT grouping of the head loads
hipError_t launch_schedule(const int32_t* kv_count, int heads, int n_qblocks, int group,
                           int n_workers, int n_groups, bool tile_order,
                           const int32_t* head_group, int32_t* lpt_order,
                           int32_t* worker_offsets, int32_t* worker_tiles,
                           int64_t* worker_load, void* ws, hipStream_t s);
int schedule_max_groups();
int schedule_max_group_heads();
// the no-allocation schedule's scratch: a static device array of
// kNoAllocScratchBytes (FVATTN_NOALLOC_SCRATCH_BYTES); *ptr = its device
// address on the current device (looked up once per device, thread-safe)
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t schedule_noalloc_scratch(void** ptr);

// ---- attn.hip --------------------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int heads, n, d, block, nb;
  float scale_log2;               // softmax scale * log2(e)
  const int32_t* kv_count;        // [heads][nb]
  const int32_t* kv_index;        // [heads][nb][nb]
  const int32_t* worker_offsets;  // null => head-major grid launch
  const int32_t* worker_tiles;
  int n_workers;
  uint64_t* timing;               // null or [n_workers][4]
  int32_t* claims;                // null or [n_workers] claim counters (run-time balancing)
  int claim_groups;               // > 1: claims only from lists w' with w' % x == w % x
  const int32_t* out_rows;        // null or [n]: result row r is stored at row out_rows[r]
  bool v_tiles;                   // V as [heads][nb][d][block] transposed tiles
  int group;                      // q-blocks per tile (1 or 2)
  int tiles_per_head;             // ceil(nb / group)
};
bool attn_has_mfma_instance(bool bf16, int d, int block);
// tiles of three q-blocks (group 3) run only on this instance set
bool attn_has_group3_instance(bool bf16, int d, int block, bool v_tiles);
// resident persistent workgroups per CU of the kernel that would run
hipError_t attn_occupancy(bool bf16, int d, int block, bool v_tiles, int group,
                          int* per_cu);
hipError_t launch_sparse_attn(const AttnArgs& a, bool bf16, hipStream_t s);

// ---- sasa.hip --------------------------------------------------------------
constexpr int kMaxSasaHeads = 4096;
constexpr int kMaxSasaGroups = 64;
size_t sasa_workspace_bytes(int heads, int n, int block, int groups);
// info: int64 [2 + 2 * groups] = mode, moves, group loads before, after
hipError_t launch_sasa_plan(const int64_t* head_load, int heads, int groups, double k1,
                            double k2, double n1, double n2, int32_t* head_group,
                            int64_t* budget, int64_t* info, hipStream_t s);
// z: the routing scores [heads][nB][nB] left by launch_route for the same inputs
hipError_t launch_sasa_augment(const float* z, int heads, int n, int block,
                               const int32_t* head_group, const int64_t* budget, int groups,
                               uint8_t* mask, int32_t* kv_count, int32_t* kv_index,
                               int64_t* head_load, float* head_density, int64_t* added,
                               void* ws, hipStream_t s);

}  // namespace fvattn
