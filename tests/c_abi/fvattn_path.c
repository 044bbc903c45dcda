/*
 * Standalone C consumer of libfvattn: one pass of the whole hot path through
 * the C ABI alone (no Python, no torch), for checking the boundary as a C
 * library.
 *
 *   fvattn_path T Y X heads d block p k_floor out_dir
 *
 * Steps: Hilbert order of the (T, Y, X) grid, Q and K gathered into that
 * order with the block mean pooling in the same pass, V packed into
 * key-block tiles, routing from the pooled means (Top-p with a Top-k floor),
 * the LPT work list, and the persistent block-sparse attention with run-time
 * claims, which stores O back in token order.  Q, K, V are bf16 values drawn
 * on the host from a fixed xorshift64* sequence.  Inputs and outputs are
 * written raw to out_dir: q.bf16, k.bf16, v.bf16, o.bf16 ([heads][n][d]),
 * perm.i32 ([n]), kv_count.i32 ([heads][nB]), kv_index.i32 ([heads][nB][nB]).
 * Exit status 0 on success; 2 on a HIP error, 3 on an fvattn error, 1 on
 * bad arguments or a file error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fvattn.h"

#define CHECK_HIP(x)                                                           \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)
#define CHECK_FV(x)                                                            \
  do {                                                                         \
    int s_ = (x);                                                              \
    if (s_ != FVATTN_OK) {                                                     \
      fprintf(stderr, "%s: %s\n", #x, fvattn_status_string(s_));               \
      exit(3);                                                                 \
    }                                                                          \
  } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static double next_uniform(void) { /* xorshift64*, 53 bits in [0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t to_bf16(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes > 0 ? bytes : 1));
  return p;
}

static void write_file(const char* dir, const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(data, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(1);
  }
  fclose(f);
}

int main(int argc, char** argv) {
  if (argc != 10) {
    fprintf(stderr, "usage: %s T Y X heads d block p k_floor out_dir\n", argv[0]);
    return 1;
  }
  const int T = atoi(argv[1]), Y = atoi(argv[2]), X = atoi(argv[3]);
  const int H = atoi(argv[4]), d = atoi(argv[5]), block = atoi(argv[6]);
  const float p = (float)atof(argv[7]);
  const int k_floor = atoi(argv[8]);
  const char* dir = argv[9];
  const int n = T * Y * X;
  if (n <= 0 || H <= 0 || d <= 0 || block <= 0) return 1;
  const int nb = (n + block - 1) / block;
  const size_t rows = (size_t)H * n * d;

  /* host inputs */
  uint16_t* hq = malloc(rows * 2);
  uint16_t* hk = malloc(rows * 2);
  uint16_t* hv = malloc(rows * 2);
  if (!hq || !hk || !hv) return 1;
  for (size_t i = 0; i < rows; ++i) hq[i] = to_bf16((float)(4.0 * next_uniform() - 2.0));
  for (size_t i = 0; i < rows; ++i) hk[i] = to_bf16((float)(4.0 * next_uniform() - 2.0));
  for (size_t i = 0; i < rows; ++i) hv[i] = to_bf16((float)(2.0 * next_uniform() - 1.0));

  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  int W = 0;
  CHECK_FV(fvattn_attn_workers(FVATTN_BF16, d, block, FVATTN_V_TILES, 2, &W));
  const int tiles = H * ((nb + 1) / 2);

  void *q = dev_alloc(rows * 2), *k = dev_alloc(rows * 2), *v = dev_alloc(rows * 2);
  void *o = dev_alloc(rows * 2), *qh = dev_alloc(rows * 2), *kh = dev_alloc(rows * 2);
  void* vt = dev_alloc((size_t)H * nb * d * block * 2);
  float* qbar = dev_alloc((size_t)H * nb * d * 4);
  float* kbar = dev_alloc((size_t)H * nb * d * 4);
  int32_t* perm = dev_alloc((size_t)n * 4);
  int32_t* inv = dev_alloc((size_t)n * 4);
  uint8_t* mask = dev_alloc((size_t)H * nb * nb);
  int32_t* kv_count = dev_alloc((size_t)H * nb * 4);
  int32_t* kv_index = dev_alloc((size_t)H * nb * nb * 4);
  int64_t* head_load = dev_alloc((size_t)H * 8);
  float* head_density = dev_alloc((size_t)H * 4);
  const size_t rws = fvattn_route_workspace_size(H, n, d, block);
  void* route_ws = dev_alloc(rws);
  int32_t* lpt_order = dev_alloc((size_t)tiles * 4);
  int32_t* worker_offsets = dev_alloc((size_t)(W + 1) * 4);
  int32_t* worker_tiles = dev_alloc((size_t)tiles * 4);
  int64_t* worker_load = dev_alloc((size_t)W * 8);
  const size_t sws = fvattn_schedule_workspace_size(H, nb, W);
  void* sched_ws = dev_alloc(sws);
  int32_t* claims = dev_alloc((size_t)W * 4);
  uint64_t* timing = dev_alloc((size_t)W * 4 * 8);
  CHECK_HIP(hipMemcpy(q, hq, rows * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, hk, rows * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, hv, rows * 2, hipMemcpyHostToDevice));

  CHECK_FV(fvattn_hilbert_permute(T, Y, X, perm, inv, s));
  CHECK_FV(fvattn_permute_pool(q, qh, perm, H, n, d, block, FVATTN_BF16, qbar, s));
  CHECK_FV(fvattn_permute_pool(k, kh, perm, H, n, d, block, FVATTN_BF16, kbar, s));
  CHECK_FV(fvattn_pack_v(v, vt, perm, H, n, d, block, FVATTN_BF16, s));
  CHECK_FV(fvattn_route_pooled(qbar, kbar, H, n, d, block, p, k_floor, mask, kv_count, kv_index,
                               head_load, head_density, route_ws, rws, s));
  CHECK_FV(fvattn_schedule(kv_count, H, nb, 2, W, 0, lpt_order, worker_offsets, worker_tiles,
                           worker_load, sched_ws, sws, s));
  CHECK_FV(fvattn_sparse_attn(qh, kh, vt, o, FVATTN_BF16, H, n, d, block, FVATTN_V_TILES, 2,
                              0.0f, kv_count, kv_index, worker_offsets, worker_tiles, W, timing,
                              claims, 0, perm, s));
  CHECK_HIP(hipStreamSynchronize(s));

  uint16_t* ho = malloc(rows * 2);
  int32_t* hperm = malloc((size_t)n * 4);
  int32_t* hcount = malloc((size_t)H * nb * 4);
  int32_t* hindex = malloc((size_t)H * nb * nb * 4);
  if (!ho || !hperm || !hcount || !hindex) return 1;
  CHECK_HIP(hipMemcpy(ho, o, rows * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hperm, perm, (size_t)n * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hcount, kv_count, (size_t)H * nb * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hindex, kv_index, (size_t)H * nb * nb * 4, hipMemcpyDeviceToHost));
  write_file(dir, "q.bf16", hq, rows * 2);
  write_file(dir, "k.bf16", hk, rows * 2);
  write_file(dir, "v.bf16", hv, rows * 2);
  write_file(dir, "o.bf16", ho, rows * 2);
  write_file(dir, "perm.i32", hperm, (size_t)n * 4);
  write_file(dir, "kv_count.i32", hcount, (size_t)H * nb * 4);
  write_file(dir, "kv_index.i32", hindex, (size_t)H * nb * nb * 4);
  printf("fvattn_path: n=%d heads=%d d=%d block=%d workers=%d ok\n", n, H, d, block, W);

  void* bufs[] = {q, k, v, o, qh, kh, vt, qbar, kbar, perm, inv, mask, kv_count, kv_index,
                  head_load, head_density, route_ws, lpt_order, worker_offsets, worker_tiles,
                  worker_load, sched_ws, claims, timing};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) CHECK_HIP(hipFree(bufs[i]));
  CHECK_HIP(hipStreamDestroy(s));
  free(hq); free(hk); free(hv); free(ho); free(hperm); free(hcount); free(hindex);
  return 0;
}
