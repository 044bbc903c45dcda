// C ABI: argument validation and dispatch.  Declarations and the contract of
// each entry point are in include/fvattn.h.  Validation happens on the host
// before any HIP call, so every error path is reachable without a GPU.
#include <math.h>

#include "fvattn.h"
#include "internal.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool dtype_ok(int dtype) { return dtype == FVATTN_F32 || dtype == FVATTN_BF16; }

size_t elem_size(int dtype) { return dtype == FVATTN_F32 ? 4 : 2; }

int launch_status(hipError_t e) { return e == hipSuccess ? FVATTN_OK : FVATTN_ELAUNCH; }

bool fits_int32(long long x) { return x >= 0 && x <= 0x7fffffffLL; }

int64_t nblocks(int n, int block) { return ((int64_t)n + block - 1) / block; }

}  // namespace

extern "C" {

const char* fvattn_status_string(int status) {
  switch (status) {
    case FVATTN_OK: return "ok";
    case FVATTN_EINVAL: return "invalid argument";
    case FVATTN_EUNSUPPORTED: return "unsupported configuration";
    case FVATTN_ELAUNCH: return "kernel launch failed";
    case FVATTN_EWORKSPACE: return "workspace missing or too small";
    case FVATTN_ESCRATCH: return "problem larger than the static scratch of the no-allocation call";
    default: return "unknown status";
  }
}

int fvattn_version(void) { return kVersion; }

int fvattn_hilbert_permute(int T, int Y, int X, int32_t* perm, int32_t* inv_perm,
                           hipStream_t stream) {
  if (!perm || !inv_perm) return FVATTN_EINVAL;
  if (T < 1 || Y < 1 || X < 1 || T > 1024 || Y > 1024 || X > 1024)
    return FVATTN_EINVAL;
  if (!fits_int32((long long)T * Y * X)) return FVATTN_EINVAL;
  return launch_status(fvattn::launch_hilbert(T, Y, X, perm, inv_perm, stream));
}

int fvattn_permute_rows(const void* src, void* dst, const int32_t* index, int heads,
                        int n, int d, int dtype, hipStream_t stream) {
  if (!src || !dst || !index) return FVATTN_EINVAL;
  if (!dtype_ok(dtype) || heads < 1 || n < 1 || d < 1) return FVATTN_EINVAL;
  if (src == dst) return FVATTN_EINVAL;
  if (!fits_int32((long long)n * d) || heads > 65535) return FVATTN_EINVAL;
  return launch_status(fvattn::launch_permute_rows(
      src, dst, index, heads, n, (size_t)d * elem_size(dtype), stream));
}

int fvattn_pack_v(const void* src, void* dst, const int32_t* index, int heads, int n,
                  int d, int block, int dtype, hipStream_t stream) {
  if (!src || !dst || !index) return FVATTN_EINVAL;
  if (!dtype_ok(dtype) || heads < 1 || n < 1 || d < 1 || block < 1) return FVATTN_EINVAL;
  if (src == dst) return FVATTN_EINVAL;
  if (!fits_int32((long long)n * d) || heads > 65535) return FVATTN_EINVAL;
  if (!fits_int32(nblocks(n, block) * block * (long long)d)) return FVATTN_EINVAL;
  if (dtype != FVATTN_BF16 || block % 16 != 0 || d % 8 != 0) return FVATTN_EUNSUPPORTED;
  if (nblocks(n, block) > 65535) return FVATTN_EUNSUPPORTED;
  return launch_status(fvattn::launch_pack_v(src, dst, index, heads, n, d, block, stream));
}

size_t fvattn_route_workspace_size(int heads, int n, int d, int block) {
  if (heads < 1 || n < 1 || d < 1 || block < 1) return 0;
  return fvattn::route_workspace_bytes(heads, n, d, block);
}

int fvattn_route(const void* q, const void* k, int dtype, int heads, int n, int d,
                 int block, float p, int k_floor, uint8_t* mask, int32_t* kv_count,
                 int32_t* kv_index, int64_t* head_load, float* head_density,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !mask || !kv_count || !kv_index || !head_load || !head_density)
    return FVATTN_EINVAL;
  if (!dtype_ok(dtype) || heads < 1 || n < 1 || d < 1 || block < 1) return FVATTN_EINVAL;
  if (!(p > 0.f) || isnan(p) || k_floor < 0) return FVATTN_EINVAL;
  if (!fits_int32((long long)n * d) || heads > 65535) return FVATTN_EINVAL;
  const int64_t nb = nblocks(n, block);
  if (d > 256 || (dtype == FVATTN_BF16 ? d % 8 : d % 4) != 0) return FVATTN_EUNSUPPORTED;
  if (nb > 4096) return FVATTN_EUNSUPPORTED;
  const size_t need = fvattn::route_workspace_bytes(heads, n, d, block);
  if (!workspace || workspace_bytes < need) return FVATTN_EWORKSPACE;
  const fvattn::RouteWorkspace ws = fvattn::route_carve(workspace, heads, n, d, block);
  return launch_status(fvattn::launch_route(q, k, dtype == FVATTN_BF16, heads, n, d, block,
                                            p, k_floor, mask, kv_count, kv_index,
                                            head_load, head_density, ws, stream));
}

int fvattn_permute_pool(const void* src, void* dst, const int32_t* index, int heads, int n,
                        int d, int block, int dtype, float* pooled, hipStream_t stream) {
  if (!src || !dst || !index || !pooled) return FVATTN_EINVAL;
  if (!dtype_ok(dtype) || heads < 1 || n < 1 || d < 1 || block < 1) return FVATTN_EINVAL;
  if (src == dst) return FVATTN_EINVAL;
  if (!fits_int32((long long)n * d) || heads > 65535) return FVATTN_EINVAL;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return FVATTN_EINVAL;
  if (d > 256 || (dtype == FVATTN_BF16 ? d % 8 : d % 4) != 0) return FVATTN_EUNSUPPORTED;
  return launch_status(fvattn::launch_permute_pool(src, dst, index, dtype == FVATTN_BF16, heads,
                                                   n, d, block, pooled, stream));
}

int fvattn_route_pooled(const float* qbar, const float* kbar, int heads, int n, int d,
                        int block, float p, int k_floor, uint8_t* mask, int32_t* kv_count,
                        int32_t* kv_index, int64_t* head_load, float* head_density,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!qbar || !kbar || !mask || !kv_count || !kv_index || !head_load || !head_density)
    return FVATTN_EINVAL;
  if (heads < 1 || n < 1 || d < 1 || block < 1) return FVATTN_EINVAL;
  if (!(p > 0.f) || isnan(p) || k_floor < 0) return FVATTN_EINVAL;
  if (!fits_int32((long long)n * d) || heads > 65535) return FVATTN_EINVAL;
  const int64_t nb = nblocks(n, block);
  if (d > 256 || d % 4 != 0) return FVATTN_EUNSUPPORTED;
  if (nb > 4096) return FVATTN_EUNSUPPORTED;
  const size_t need = fvattn::route_workspace_bytes(heads, n, d, block);
  if (!workspace || workspace_bytes < need) return FVATTN_EWORKSPACE;
  const fvattn::RouteWorkspace ws = fvattn::route_carve(workspace, heads, n, d, block);
  return launch_status(fvattn::launch_route_pooled(qbar, kbar, heads, n, d, block, p, k_floor,
                                                   mask, kv_count, kv_index, head_load,
                                                   head_density, ws, stream));
}

size_t fvattn_schedule_workspace_size(int heads, int n_qblocks, int n_workers) {
  if (heads < 1 || n_qblocks < 1 || n_workers < 1) return 0;
  return fvattn::schedule_workspace_bytes(heads, n_qblocks, n_workers);
}

int fvattn_schedule(const int32_t* kv_count, int heads, int n_qblocks, int group,
                    int n_workers, int flags, int32_t* lpt_order, int32_t* worker_offsets,
                    int32_t* worker_tiles, int64_t* worker_load, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (!kv_count || !lpt_order || !worker_offsets || !worker_tiles || !worker_load)
    return FVATTN_EINVAL;
  if (heads < 1 || n_qblocks < 1 || n_workers < 1) return FVATTN_EINVAL;
  if (group < 1 || group > 3) return FVATTN_EINVAL;
  if (!fits_int32((long long)heads * n_qblocks)) return FVATTN_EINVAL;
  if (flags & ~(FVATTN_SCHED_TILE_ORDER | FVATTN_SCHED_GROUPS(0xFF))) return FVATTN_EINVAL;
  if (n_workers > fvattn::kMaxWorkers) return FVATTN_EUNSUPPORTED;
  const int n_groups = (flags >> 8) & 0xFF;
  if (n_groups > 1) {
    if (n_groups > fvattn::schedule_max_groups() || n_groups > n_workers) return FVATTN_EINVAL;
    if (heads > fvattn::schedule_max_group_heads()) return FVATTN_EUNSUPPORTED;
  }
  const size_t need = fvattn::schedule_workspace_bytes(heads, n_qblocks, n_workers);
  if (!workspace || workspace_bytes < need) return FVATTN_EWORKSPACE;
  return launch_status(fvattn::launch_schedule(
      kv_count, heads, n_qblocks, group, n_workers, n_groups > 1 ? n_groups : 1,
      (flags & FVATTN_SCHED_TILE_ORDER) != 0, nullptr,
      lpt_order, worker_offsets, worker_tiles, worker_load, workspace, stream));
}

int fvattn_schedule_noalloc(const int32_t* kv_count, int heads, int n_qblocks, int group,
                            int n_workers, int flags, int32_t* lpt_order,
                            int32_t* worker_offsets, int32_t* worker_tiles,
                            int64_t* worker_load, hipStream_t stream) {
  static_assert(fvattn::kNoAllocScratchBytes == FVATTN_NOALLOC_SCRATCH_BYTES, "scratch size");
  if (!kv_count || !lpt_order || !worker_offsets || !worker_tiles || !worker_load)
    return FVATTN_EINVAL;
  if (heads < 1 || n_qblocks < 1 || n_workers < 1) return FVATTN_EINVAL;
  if (group < 1 || group > 3) return FVATTN_EINVAL;
  if (!fits_int32((long long)heads * n_qblocks)) return FVATTN_EINVAL;
  if (flags & ~(FVATTN_SCHED_TILE_ORDER | FVATTN_SCHED_GROUPS(0xFF))) return FVATTN_EINVAL;
  if (n_workers > fvattn::kMaxWorkers) return FVATTN_EUNSUPPORTED;
  const int n_groups = (flags >> 8) & 0xFF;
  if (n_groups > 1) {
    if (n_groups > fvattn::schedule_max_groups() || n_groups > n_workers) return FVATTN_EINVAL;
    if (heads > fvattn::schedule_max_group_heads()) return FVATTN_EUNSUPPORTED;
  }
  // the size check comes before any HIP call, so it holds without a device
  if (fvattn::schedule_workspace_bytes(heads, n_qblocks, n_workers) >
      fvattn::kNoAllocScratchBytes)
    return FVATTN_ESCRATCH;
  void* ws = nullptr;
  if (fvattn::schedule_noalloc_scratch(&ws) != hipSuccess) return FVATTN_ELAUNCH;
  return launch_status(fvattn::launch_schedule(
      kv_count, heads, n_qblocks, group, n_workers, n_groups > 1 ? n_groups : 1,
      (flags & FVATTN_SCHED_TILE_ORDER) != 0, nullptr,
      lpt_order, worker_offsets, worker_tiles, worker_load, ws, stream));
}

int fvattn_schedule_heads(const int32_t* kv_count, int heads, int n_qblocks, int group,
                          int n_workers, int n_groups, const int32_t* head_group, int flags,
                          int32_t* lpt_order, int32_t* worker_offsets, int32_t* worker_tiles,
                          int64_t* worker_load, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!kv_count || !head_group || !lpt_order || !worker_offsets || !worker_tiles ||
      !worker_load)
    return FVATTN_EINVAL;
  if (heads < 1 || n_qblocks < 1 || n_workers < 1) return FVATTN_EINVAL;
  if (group < 1 || group > 3) return FVATTN_EINVAL;
  if (!fits_int32((long long)heads * n_qblocks)) return FVATTN_EINVAL;
  if (flags & ~FVATTN_SCHED_TILE_ORDER) return FVATTN_EINVAL;
  if (n_groups < 2 || n_groups > fvattn::schedule_max_groups() || n_groups > n_workers)
    return FVATTN_EINVAL;
  if (n_workers > fvattn::kMaxWorkers) return FVATTN_EUNSUPPORTED;
  const size_t need = fvattn::schedule_workspace_bytes(heads, n_qblocks, n_workers);
  if (!workspace || workspace_bytes < need) return FVATTN_EWORKSPACE;
  return launch_status(fvattn::launch_schedule(
      kv_count, heads, n_qblocks, group, n_workers, n_groups,
      (flags & FVATTN_SCHED_TILE_ORDER) != 0, head_group,
      lpt_order, worker_offsets, worker_tiles, worker_load, workspace, stream));
}

int fvattn_sasa_plan(const int64_t* head_load, int heads, int n_groups, double k1, double k2,
                     double n1, double n2, int32_t* head_group, int64_t* group_budget,
                     int64_t* info, hipStream_t stream) {
  if (!head_load || !head_group || !group_budget || !info) return FVATTN_EINVAL;
  if (heads < 1 || n_groups < 1) return FVATTN_EINVAL;
  if (!(k1 >= 1.0) || !(k2 >= k1) || isinf(k2) || !(n1 >= 0.0) || !(n1 <= 1.0) ||
      !(n2 >= 0.0) || !(n2 <= 1.0))
    return FVATTN_EINVAL;
  if (heads > fvattn::kMaxSasaHeads || n_groups > fvattn::kMaxSasaGroups)
    return FVATTN_EUNSUPPORTED;
  return launch_status(fvattn::launch_sasa_plan(head_load, heads, n_groups, k1, k2, n1, n2,
                                                head_group, group_budget, info, stream));
}

size_t fvattn_sasa_workspace_size(int heads, int n, int block, int n_groups) {
  if (heads < 1 || n < 1 || block < 1 || n_groups < 1) return 0;
  return fvattn::sasa_workspace_bytes(heads, n, block, n_groups);
}

int fvattn_sasa_augment(const void* route_workspace, size_t route_workspace_bytes, int heads,
                        int n, int d, int block, const int32_t* head_group,
                        const int64_t* group_budget, int n_groups, uint8_t* mask,
                        int32_t* kv_count, int32_t* kv_index, int64_t* head_load,
                        float* head_density, int64_t* added, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (!route_workspace || !head_group || !group_budget || !mask || !kv_count || !kv_index ||
      !head_load || !head_density || !added)
    return FVATTN_EINVAL;
  if (heads < 1 || n < 1 || d < 1 || block < 1 || n_groups < 1) return FVATTN_EINVAL;
  if (!fits_int32((long long)n * d) || heads > 65535) return FVATTN_EINVAL;
  const int64_t nb = nblocks(n, block);
  if (nb > 4096) return FVATTN_EUNSUPPORTED;
  if (n_groups > fvattn::kMaxSasaGroups) return FVATTN_EUNSUPPORTED;
  if (route_workspace_bytes < fvattn::route_workspace_bytes(heads, n, d, block))
    return FVATTN_EWORKSPACE;
  const size_t need = fvattn::sasa_workspace_bytes(heads, n, block, n_groups);
  if (!workspace || workspace_bytes < need) return FVATTN_EWORKSPACE;
  const fvattn::RouteWorkspace rw =
      fvattn::route_carve(const_cast<void*>(route_workspace), heads, n, d, block);
  return launch_status(fvattn::launch_sasa_augment(rw.z, heads, n, block, head_group,
                                                   group_budget, n_groups, mask, kv_count,
                                                   kv_index, head_load, head_density, added,
                                                   workspace, stream));
}

int fvattn_sparse_attn(const void* q, const void* k, const void* v, void* o, int dtype,
                       int heads, int n, int d, int block, int v_layout, int group,
                       float scale,
                       const int32_t* kv_count, const int32_t* kv_index,
                       const int32_t* worker_offsets, const int32_t* worker_tiles,
                       int n_workers, uint64_t* timing, int32_t* claims, int claim_groups,
                       const int32_t* out_rows, hipStream_t stream) {
  if (!q || !k || !v || !o || !kv_count || !kv_index) return FVATTN_EINVAL;
  if (!dtype_ok(dtype) || heads < 1 || n < 1 || d < 1 || block < 1) return FVATTN_EINVAL;
  if (isnan(scale) || isinf(scale)) return FVATTN_EINVAL;
  if (v_layout != FVATTN_V_ROWS && v_layout != FVATTN_V_TILES) return FVATTN_EINVAL;
  if (group < 1 || group > 3) return FVATTN_EINVAL;
  if (!fits_int32((long long)n * d) || heads > 65535) return FVATTN_EINVAL;
  const int64_t nb = nblocks(n, block);
  if (!fits_int32((long long)heads * nb) || !fits_int32(nb * nb)) return FVATTN_EINVAL;
  if (worker_offsets) {
    if (!worker_tiles || n_workers < 1) return FVATTN_EINVAL;
  }
  const bool bf16 = dtype == FVATTN_BF16;
  if (!fvattn::attn_has_mfma_instance(bf16, d, block) && (d > 128 || block > 256))
    return FVATTN_EUNSUPPORTED;
  // the tiled-V kernels address one head of K and of V at a time with 32-bit
  // byte offsets; tiles exist only for blocks of a multiple of 16 rows
  // (fvattn_pack_v)
  if (v_layout == FVATTN_V_TILES &&
      ((long long)nb * block * d * 2 > 0xffffffffLL || block % 16 != 0))
    return FVATTN_EUNSUPPORTED;
  if ((timing || claims) && !worker_offsets) return FVATTN_EINVAL;
  if (claim_groups < 0 || claim_groups > 64) return FVATTN_EINVAL;
  // three q-blocks per tile: bf16 V tiles of 128-key blocks, d 64 or 128
  if (group == 3 &&
      !fvattn::attn_has_group3_instance(bf16, d, block, v_layout == FVATTN_V_TILES))
    return FVATTN_EUNSUPPORTED;
  fvattn::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.heads = heads;
  a.n = n;
  a.d = d;
  a.block = block;
  a.nb = (int)nb;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.kv_count = kv_count;
  a.kv_index = kv_index;
  a.worker_offsets = worker_offsets;
  a.worker_tiles = worker_tiles;
  a.n_workers = worker_offsets ? n_workers : 0;
  a.timing = timing;
  a.claims = claims;
  a.claim_groups = claim_groups;
  a.out_rows = out_rows;
  a.v_tiles = v_layout == FVATTN_V_TILES;
  a.group = group;
  a.tiles_per_head = (int)((nb + group - 1) / group);
  return launch_status(fvattn::launch_sparse_attn(a, bf16, stream));
}

int fvattn_attn_workers(int dtype, int d, int block, int v_layout, int group,
                        int* workers) {
  if (!workers || !dtype_ok(dtype) || d < 1 || block < 1) return FVATTN_EINVAL;
  if (v_layout != FVATTN_V_ROWS && v_layout != FVATTN_V_TILES) return FVATTN_EINVAL;
  if (group < 1 || group > 3) return FVATTN_EINVAL;
  if (group == 3 && !fvattn::attn_has_group3_instance(dtype == FVATTN_BF16, d, block,
                                                      v_layout == FVATTN_V_TILES))
    return FVATTN_EUNSUPPORTED;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FVATTN_ELAUNCH;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return FVATTN_ELAUNCH;
  if (fvattn::attn_occupancy(dtype == FVATTN_BF16, d, block, v_layout == FVATTN_V_TILES,
                             group, &per_cu) != hipSuccess)
    return FVATTN_ELAUNCH;
  *workers = cus * (per_cu > 0 ? per_cu : 1);
  return FVATTN_OK;
}

}  // extern "C"
