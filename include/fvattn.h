/*
 * fvattn.h - C ABI of the MI355X (gfx950) FVAttn single-GPU hot path.
 *
 * The method (FVAttn, "Adaptive Sparse Attention with Runtime Load Balancing
 * for Video Generation"; arXiv abstract on the mlsanity.com index page):
 * order the spatio-temporal token grid along a Hilbert curve, route each query
 * block to the key blocks that matter with a Top-p threshold and a Top-k
 * floor computed from pooled Q/K, and run attention over the kept blocks only.
 * The pages balance the resulting uneven per-head work across GPU ranks; this
 * library balances it across the workgroups of one GPU with an LPT work list
 * that feeds a persistent attention kernel.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors Q, K, V, O are contiguous row-major [heads][n][d] in device
 *    memory; a batch (or guidance copy) is folded into `heads`.
 *  - Blocks: block j holds rows [j*block, min(n, (j+1)*block)); the last one
 *    may be short.  nB = ceil(n / block).  Tile t = h * nB + i is query
 *    block i of head h.
 *  - dtype: FVATTN_F32 (float) or FVATTN_BF16 (bfloat16 storage, fp32
 *    accumulation).
 *  - Ownership: the caller allocates every buffer (outputs and workspace) and
 *    keeps it alive until the stream work is done.  The library never
 *    allocates, frees or caches device memory; it is re-entrant.  The one
 *    piece of global state is the static scratch array of
 *    fvattn_schedule_noalloc (one per GPU, for callers that cannot
 *    allocate).
 *  - Streams: every call only enqueues kernels on `stream` (0 = the null
 *    stream) and returns; it never synchronises the host.
 *  - Errors: arguments are validated on the host before anything is
 *    launched; a failed check returns a negative status and launches nothing.
 *    A failed launch returns FVATTN_ELAUNCH.  Faults inside a kernel surface
 *    at the caller's next synchronisation.
 */
#ifndef FVATTN_H
#define FVATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FVATTN_OK 0
#define FVATTN_EINVAL (-1)       /* bad pointer, size or parameter            */
#define FVATTN_EUNSUPPORTED (-2) /* valid, but no kernel instance for it     */
#define FVATTN_ELAUNCH (-3)      /* the HIP launch itself failed             */
#define FVATTN_EWORKSPACE (-4)   /* workspace pointer null or too small      */
#define FVATTN_ESCRATCH (-5)     /* larger than the static scratch of the
                                    no-allocation call                       */

/* Storage types. */
#define FVATTN_F32 0
#define FVATTN_BF16 1

/* fvattn_schedule flags. */
#define FVATTN_SCHED_TILE_ORDER 1
/* two-level LPT over x worker groups (2 <= x <= 64), see fvattn_schedule */
#define FVATTN_SCHED_GROUPS(x) ((x) << 8)

/* V layouts accepted by fvattn_sparse_attn. */
#define FVATTN_V_ROWS 0    /* [heads][n][d], like Q and K                     */
#define FVATTN_V_TILES 1   /* [heads][nB][d][block]: one transposed tile per
                              key block, padding keys zero (fvattn_pack_v)   */

/* Static string naming a status code. */
const char* fvattn_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fvattn_version(void);

/*
 * Hilbert order of a T x Y x X token grid.
 *
 * Source: the routing frontend regroups tokens along a Hilbert curve so that
 * spatially close tokens fall into the same or neighbouring blocks (aixai.ru
 * FVAttn post, section "Sparse-routing frontend"; PaperDaily FVAttn article,
 * method section).  Curve: J. Skilling's 3D construction on the enclosing
 * cube of side 2^b, b = max(1, ceil(log2(max(T, Y, X)))), axis order (t, y, x),
 * index bits interleaved MSB first with t on top; grid points are ranked by
 * their index on that cube.
 *
 * Token n = (t*Y + y)*X + x.  Outputs (device, int32[T*Y*X] each):
 *   perm[r]          = token at Hilbert rank r,
 *   inv_perm[perm[r]] = r.
 * Limits: 1 <= T, Y, X <= 1024 and T*Y*X < 2^31; otherwise FVATTN_EINVAL.
 */
int fvattn_hilbert_permute(int T, int Y, int X, int32_t* perm,
                           int32_t* inv_perm, hipStream_t stream);

/*
 * Row gather, used to put Q/K/V into Hilbert order and O back:
 *   dst[h][r][:] = src[h][index[r]][:]   for h < heads, r < n.
 * index: device int32[n], every entry in [0, n) (not checked on the device).
 * src and dst must not overlap.  d >= 1.
 */
int fvattn_permute_rows(const void* src, void* dst, const int32_t* index,
                        int heads, int n, int d, int dtype,
                        hipStream_t stream);

/*
 * Row gather into transposed key-block tiles, used for V (FVATTN_V_TILES):
 *   tile (h, j) row c holds column c of rows index[j*block + r] of src[h],
 *   r = 0 .. block-1, with 0 for the padding rows of the last block.  Each
 *   tile row is stored in 8-byte units of 4 consecutive r; inside every group
 *   of 16 keys the four units are stored in the order 0, 2, 1, 3, so that the
 *   8 keys one lane of the attention kernel's 32x32x16 MFMA takes ({4g..4g+3}
 *   and {8+4g..8+4g+3} of the group, g = 0, 1) are 16 contiguous bytes.  So
 *   element (h, j, c, r) is at ((h*nB + j)*d + c)*block + pos(r), with
 *   pos(r) = 16*(r/16) + 4*sigma((r%16)/4) + r%4, sigma = (0, 2, 1, 3).
 * dst holds heads * nB * d * block elements.  The attention kernels read
 * V^T as the A operand of the P.V product; producing it inside the Hilbert
 * gather costs no extra memory traffic.
 * bf16 only; block % 16 == 0, d % 8 == 0 (else FVATTN_EUNSUPPORTED).
 */
int fvattn_pack_v(const void* src, void* dst, const int32_t* index, int heads,
                  int n, int d, int block, int dtype, hipStream_t stream);

/*
 * Routing: block importance from mean-pooled Q/K, Top-p cut, Top-k floor.
 *
 * Source: importance of key blocks is estimated from pooled Q and K, and one
 * routing pass yields the mask and each head's density (PaperDaily FVAttn
 * article, method section; aixai.ru post, "Sparse-routing frontend"); Top-p
 * keeps blocks in importance order until their accumulated importance
 * reaches p (aixai.ru post, "Top-p vs Top-k"); the Top-k floor always keeps
 * the k most important ones (PaperDaily article, method section).
 *
 * Computed, on Hilbert-ordered q, k [heads][n][d]:
 *   qbar[h][i] = mean of q rows of block i (true row count), same for kbar;
 *   z[h][i][j] = qbar[h][i] . kbar[h][j] / sqrt(d);
 *   P[h][i][:] = softmax_j z[h][i][:];
 *   blocks ranked by (P descending, j ascending); n_p = smallest prefix whose
 *   accumulated P is >= p (nB if p >= 1 or if none reaches p);
 *   n_keep = min(nB, max(n_p, k_floor)).
 * Outputs (device):
 *   mask        uint8 [heads][nB][nB], 1 = kept;
 *   kv_count    int32 [heads][nB] = n_keep;
 *   kv_index    int32 [heads][nB][nB], kept j ascending in the first
 *               kv_count entries of each row (the rest is left untouched);
 *   head_load   int64 [heads] = sum_i kv_count[h][i];
 *   head_density float [heads] = head_load / nB^2.
 * Arithmetic is fp32 on the device (pooling, scores, softmax, prefix sums).
 * Limits: d <= 256 and d % 8 == 0 (bf16) or d % 4 == 0 (f32); nB <= 4096;
 * 0 < p (p >= 1 keeps everything); k_floor >= 0.
 * workspace: device memory of at least fvattn_route_workspace_size() bytes.
 */
size_t fvattn_route_workspace_size(int heads, int n, int d, int block);
int fvattn_route(const void* q, const void* k, int dtype, int heads, int n,
                 int d, int block, float p, int k_floor, uint8_t* mask,
                 int32_t* kv_count, int32_t* kv_index, int64_t* head_load,
                 float* head_density, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * Gather into Hilbert order fused with the routing's mean pooling: one read
 * of the tensor gives both the reordered rows and the pooled block means
 * (PaperDaily FVAttn article, method section: blocks formed along the Hilbert
 * curve, importance from pooled Q/K; the overlap and fusion that keeps such
 * bookkeeping off the critical path is in its section on the implementation
 * and in the "Key findings" of the wiki post "FVAttn: Adaptive Sparse Attention
 * with Runtime Load Balancing").
 *
 * Computed, for src [heads][n][d] (bf16 or f32, device), index int32[n]:
 *   dst[h][r][:] = src[h][index[r]][:]            (as fvattn_permute_rows)
 *   pooled[h][j][c] = mean over the rows r of block j (r < n) of dst[h][r][c]
 * pooled is fp32 [heads][nB][d], nB = ceil(n / block), caller-owned device
 * memory; its values equal, bit for bit, the pooled means fvattn_route
 * computes from dst (the same fp32 summation order).
 * src and dst: 16-byte aligned, distinct (else FVATTN_EINVAL); limits as for
 * fvattn_route: d <= 256, d % 8 == 0 (bf16) or d % 4 == 0 (f32), else
 * FVATTN_EUNSUPPORTED.  Asynchronous on `stream`.
 */
int fvattn_permute_pool(const void* src, void* dst, const int32_t* index, int heads, int n,
                        int d, int block, int dtype, float* pooled, hipStream_t stream);

/*
 * fvattn_route from given pooled means: qbar, kbar fp32 [heads][nB][d]
 * (device; what fvattn_permute_pool writes for Q and K).  Everything after
 * the pooling is the same computation, with the same outputs, limits
 * (d % 4 == 0 here) and errors as fvattn_route.  workspace: at least
 * fvattn_route_workspace_size(heads, n, d, block) bytes; the scores land in
 * it where fvattn_route puts them, so fvattn_sasa_augment can read them.
 */
int fvattn_route_pooled(const float* qbar, const float* kbar, int heads, int n, int d,
                        int block, float p, int k_floor, uint8_t* mask, int32_t* kv_count,
                        int32_t* kv_index, int64_t* head_load, float* head_density,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * LPT work list over tiles for n_workers persistent workgroups.  A tile is
 * `group` consecutive q-blocks of one head (group 1, 2 or 3): tile
 * t = h * ceil(n_qblocks / group) + m covers q-blocks [m*group,
 * min(n_qblocks, (m+1)*group)).  group 2 and 3 match the attention kernels
 * that load each K/V block once for two or three q-blocks.
 *
 * Source: once the mask exists each head's load in sparse blocks is known
 * exactly and a few heavy heads set the critical path (aixai.ru FVAttn post,
 * section "Runtime Load Balancing (RLB)").  On one GPU the balanced resource
 * is the set of workgroups; the rule is Graham's LPT:
 *   cost(t) = sum of kv_count over the tile's q-blocks;
 *   lpt_order = tiles sorted by (cost descending, t ascending);
 *   in that order each tile goes to the worker with the least load so far
 *   (lowest worker index on ties) and is appended to its list.
 * Outputs (device), with tiles = heads * ceil(n_qblocks / group):
 *   lpt_order      int32 [tiles];
 *   worker_offsets int32 [n_workers+1], exclusive prefix of list sizes;
 *   worker_tiles   int32 [tiles], the lists concatenated;
 *   worker_load    int64 [n_workers], summed cost per worker.
 * flags:
 *   0                        each list in assignment order;
 *   FVATTN_SCHED_TILE_ORDER  each list sorted by ascending tile id.  Same
 *                            assignment and loads; a persistent kernel then
 *                            walks heads in step across workgroups, so K/V
 *                            blocks are shared in L2 while they run.
 *   FVATTN_SCHED_GROUPS(x)   two-level LPT, the single-GPU image of the
 *                            pages' balancing of heavy heads between ranks:
 *                            worker w belongs to group w % x (x = the XCD
 *                            count makes a group one XCD, since persistent
 *                            workgroup w runs on XCD w % 8 on MI355X); head
 *                            loads (sums of their tile costs) go to the
 *                            groups by the same LPT rule (heads by (load
 *                            desc, head asc), least-loaded group, lowest
 *                            index on ties); then each tile, in lpt_order,
 *                            goes to the least-loaded worker of its head's
 *                            group (lowest index on ties).  Every head's
 *                            K/V then stays in one XCD's L2.  x <= 64 and
 *                            x <= n_workers (else FVATTN_EINVAL); heads <=
 *                            4096 (else FVATTN_EUNSUPPORTED).  Combines
 *                            with FVATTN_SCHED_TILE_ORDER.
 * Bit-exact: there is exactly one correct result per input and flag.
 * Limits: 1 <= n_workers <= 2048; tile costs are clamped to [0, 65535];
 * heads*n_qblocks < 2^31; group in {1, 2, 3} (else FVATTN_EINVAL).
 * workspace: at least fvattn_schedule_workspace_size() bytes.
 */
size_t fvattn_schedule_workspace_size(int heads, int n_qblocks, int n_workers);
int fvattn_schedule(const int32_t* kv_count, int heads, int n_qblocks,
                    int group, int n_workers, int flags, int32_t* lpt_order,
                    int32_t* worker_offsets, int32_t* worker_tiles,
                    int64_t* worker_load, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * fvattn_schedule for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, outputs, limits and errors as fvattn_schedule, except that
 * there is no workspace argument: the scratch is a static device array of
 * FVATTN_NOALLOC_SCRATCH_BYTES (8 MiB) that each GPU the library runs on
 * holds until the process ends.  Problems whose
 * fvattn_schedule_workspace_size(heads, n_qblocks, n_workers) exceeds it
 * return FVATTN_ESCRATCH before anything is launched (about 209k
 * heads * n_qblocks; 40 heads x 4096 q-blocks fit).  The call allocates and
 * frees nothing; the first call on a device looks up the array's device
 * address (hipGetSymbolAddress), later calls reuse it.  Nothing in the
 * scratch needs clearing between calls (every word a kernel reads was
 * written earlier in the same call).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (two streams, or two
 * host threads) race and give undefined results; order them on one stream.
 * Outputs equal fvattn_schedule's bit for bit.
 */
#define FVATTN_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int fvattn_schedule_noalloc(const int32_t* kv_count, int heads, int n_qblocks,
                            int group, int n_workers, int flags, int32_t* lpt_order,
                            int32_t* worker_offsets, int32_t* worker_tiles,
                            int64_t* worker_load, hipStream_t stream);

/*
 * Two-level LPT with the head -> group map given: as fvattn_schedule with
 * FVATTN_SCHED_GROUPS(n_groups), except that head h belongs to group
 * head_group[h] (device int32 [heads], values clamped to [0, n_groups))
 * instead of the LPT grouping of the head loads.  This is the schedule of
 * the per-rank image of fvattn_sasa_plan (groups = ranks, heads sharded,
 * then moved by the plan).  flags: 0 or FVATTN_SCHED_TILE_ORDER;
 * 2 <= n_groups <= min(64, n_workers).  Other limits, outputs, workspace and
 * errors as fvattn_schedule.  Bit-exact.
 */
int fvattn_schedule_heads(const int32_t* kv_count, int heads, int n_qblocks,
                          int group, int n_workers, int n_groups,
                          const int32_t* head_group, int flags, int32_t* lpt_order,
                          int32_t* worker_offsets, int32_t* worker_tiles,
                          int64_t* worker_load, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Slack-aware sparse augmentation (SASA), planning step.
 *
 * Source: after balancing, ranks off the critical path wait for it; SASA
 * spends that idle time on extra high-value blocks on those ranks only, and
 * the imbalance factor selects the regime with thresholds k1 = 1.05 and
 * k2 = 1.10 (nothing below k1, SASA alone below k2, runtime load balancing
 * (RLB) and then SASA above), with an augmentation coefficient n1 = 0.8 and
 * a trigger threshold n2 = 0.07; RLB moves at most one local head per rank
 * (aixai.ru FVAttn post, sections "Runtime Load Balancing (RLB)" and
 * "Slack-Aware Sparse Augmentation (SASA)"; PaperDaily FVAttn article, SASA
 * paragraphs).  On one GPU the ranks are n_groups groups of persistent
 * workers (worker w in group w % n_groups; 8 = one per XCD on MI355X):
 *   start:  head h in group floor(h * n_groups / heads) (contiguous shards);
 *   loads:  group load = sum of head_load over its heads (kept blocks);
 *           rho = max / mean of the group loads (float64);
 *   mode:   0 if rho < k1, 1 (SASA) if rho < k2, else 2 (RLB + SASA);
 *   RLB (mode 2): while the critical group (largest load, lowest index) has
 *           given no head, move its heaviest head not moved before (lowest
 *           index on ties) with load > 0 and load_t + load_h < load_c to the
 *           least-loaded group t (lowest index); stop when there is none;
 *   budget (modes 1, 2): slack_g = max load - load_g; group_budget[g] =
 *           floor(n1 * slack_g) if slack_g >= n2 * max load (float64), else 0.
 * Inputs: head_load (device int64 [heads], as fvattn_route writes it).
 * Outputs (device): head_group int32 [heads]; group_budget int64 [n_groups]
 * (extra blocks per group); info int64 [2 + 2*n_groups] = mode, number of
 * head moves, group loads before the moves, group loads after.
 * Bit-exact (integer arithmetic and float64 comparisons).
 * Errors: FVATTN_EINVAL for null pointers, heads or n_groups < 1, k1 < 1,
 * k2 < k1 or infinite, n1 or n2 outside [0, 1]; FVATTN_EUNSUPPORTED for
 * heads > 4096 or n_groups > 64.
 */
int fvattn_sasa_plan(const int64_t* head_load, int heads, int n_groups,
                     double k1, double k2, double n1, double n2,
                     int32_t* head_group, int64_t* group_budget, int64_t* info,
                     hipStream_t stream);

/*
 * SASA augmentation: adds to the mask, for every group g with
 * group_budget[g] > 0, the group_budget[g] blocks it skipped whose routing
 * importance is largest (all of them if there are fewer), and rewrites the
 * routing outputs to match.
 *
 * Source: the extra blocks come from the blocks the sparse mask skipped, in
 * importance order, and the routing pass already gives that order (aixai.ru
 * FVAttn post, sections "Sparse-routing frontend" and "Slack-Aware Sparse
 * Augmentation (SASA)"; PaperDaily FVAttn article).  Importance of (h, i, j)
 * = the routing softmax P[h][i][j] = exp(z - max z) / sum, recomputed in
 * fp32 from the scores fvattn_route leaves in its workspace, with the
 * routing pass's own arithmetic; blocks of a group are ranked by (P desc,
 * h asc, i asc, j asc) over the group's heads (head_group[h]).
 * route_workspace: the workspace of the fvattn_route call that produced
 *   mask/kv_* for the same (heads, n, d, block), unchanged since.
 * In/out (device): mask, kv_count, kv_index (ascending, as fvattn_route
 *   writes them); head_load and head_density are recomputed for every head.
 * Out: added int64 [n_groups], blocks added per group.
 * workspace: at least fvattn_sasa_workspace_size(heads, n, block, n_groups).
 * Errors: FVATTN_EINVAL for null pointers or bad sizes; FVATTN_EUNSUPPORTED
 * for nB > 4096 or n_groups > 64; FVATTN_EWORKSPACE for a short workspace.
 * Rows of groups without a budget are left untouched.
 */
size_t fvattn_sasa_workspace_size(int heads, int n, int block, int n_groups);
int fvattn_sasa_augment(const void* route_workspace, size_t route_workspace_bytes,
                        int heads, int n, int d, int block,
                        const int32_t* head_group, const int64_t* group_budget,
                        int n_groups, uint8_t* mask, int32_t* kv_count,
                        int32_t* kv_index, int64_t* head_load, float* head_density,
                        int64_t* added, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Block-sparse attention over the kept blocks.
 *
 * Source: only the (query block, key block) pairs the routing keeps are
 * computed (aixai.ru FVAttn post, "What is sparse attention in video
 * transformers"; arXiv abstract).  For each tile (h, i):
 *   O[h][rows of block i] = softmax(Q_i K_S^T * scale) V_S,
 * S = the rows of the blocks kv_index[h][i][0 .. kv_count[h][i]).  No causal
 * mask.  fp32 accumulation; O is stored in dtype.  A row with kv_count 0 is
 * written as zeros.
 *
 * scale <= 0 selects 1/sqrt(d).
 * v_layout: FVATTN_V_ROWS or FVATTN_V_TILES (see fvattn_pack_v); Q, K and O
 * are always [heads][n][d].  With FVATTN_V_TILES one head of V tiles
 * (nB * block * d elements) must fit in 4 GiB and block % 16 == 0 (else
 * FVATTN_EUNSUPPORTED); the tensors themselves have no size limit beyond
 * n * d < 2^31.
 * kv_index entries must lie in [0, nB): the MFMA kernels clamp others into
 * that range, the plain kernel skips them (memory-safe, result undefined).
 * kv_count entries above nB count as nB; entries of 0 or below leave the
 * q-block's rows zero.
 * Work distribution (tiles of `group` q-blocks, numbered as in
 * fvattn_schedule; group 2 with FVATTN_V_TILES and an MFMA shape runs the
 * kernel that shares each K/V block between the two q-blocks; group 3, the
 * same for three q-blocks, three wavefronts per SIMD, exists for bf16
 * FVATTN_V_TILES with block 128 and d 64 or 128 only, else
 * FVATTN_EUNSUPPORTED):
 *   worker_offsets != NULL: persistent launch of n_workers workgroups;
 *     workgroup w runs the tiles worker_tiles[worker_offsets[w] ..
 *     worker_offsets[w+1]) in order (the LPT lists of fvattn_schedule);
 *   worker_offsets == NULL: one workgroup per tile in head-major order (the
 *     unbalanced control); worker_tiles and n_workers are ignored.
 * timing (nullable, device uint64 [n_workers][4], persistent launch only):
 *   {start, end} of each workgroup on the 100 MHz constant clock
 *   (s_memrealtime), the raw HW_ID register and the XCC_ID register.
 * claims (nullable, device int32 [n_workers], persistent launch only):
 *   run-time balancing on top of the LPT lists, the single-GPU image of the
 *   pages' runtime load balancing (aixai.ru FVAttn post, "Runtime Load
 *   Balancing (RLB)"): the LPT plan predicts loads, the hardware's per-CU
 *   speed differs, so a workgroup that finishes its own list early takes the
 *   next unstarted tile of the list with the most tiles left.  claims[w]
 *   counts the tiles of list w handed out; the call resets the array (with a
 *   kernel on `stream`) and the attention kernel updates it with atomics, so
 *   the caller only owns the memory, and calls that share it must not
 *   overlap.  Every tile still runs exactly once, in one workgroup, so the
 *   output is the same bits as without claims.  Honoured by the kernels for
 *   tiles of two or three q-blocks (group 2 or 3, FVATTN_V_TILES, an MFMA
 *   shape); the other kernels run their lists as given.
 * claim_groups (0 <= x <= 64): 0 or 1 lets a workgroup claim from every
 *   list; x > 1 only from the lists w' with w' % x == w % x, so the worker
 *   groups of fvattn_schedule_heads stay independent, like ranks.
 * out_rows (nullable, device int32 [n]): result row r of every head is stored
 *   at row out_rows[r] of o instead of row r; passing the Hilbert order `perm`
 *   of fvattn_hilbert_permute writes O straight back in token order, which
 *   saves the separate inverse permute pass.  Must hold distinct rows in
 *   [0, n) (rows written twice race; out-of-range rows are not checked).
 * Kernels: bf16 with (d, block) in {(64, 64), (128, 128), (64, 128),
 * (128, 64)} runs on an MFMA kernel (the LDS-DMA ones for FVATTN_V_TILES);
 * every other (dtype, d <= 128, block <= 256) combination runs on a plain
 * fp32 VALU kernel.
 */
int fvattn_sparse_attn(const void* q, const void* k, const void* v, void* o,
                       int dtype, int heads, int n, int d, int block,
                       int v_layout, int group, float scale,
                       const int32_t* kv_count,
                       const int32_t* kv_index, const int32_t* worker_offsets,
                       const int32_t* worker_tiles, int n_workers,
                       uint64_t* timing, int32_t* claims, int claim_groups,
                       const int32_t* out_rows, hipStream_t stream);

/*
 * Persistent workers for fvattn_sparse_attn on the current device: the
 * number of workgroups of the attention kernel that (dtype, d, block,
 * v_layout, group) selects which can be resident at once (compute units times
 * workgroups per compute unit).  Pass it as n_workers to fvattn_schedule and
 * fvattn_sparse_attn so every compute unit stays busy.  Writes *workers;
 * returns FVATTN_EINVAL for bad arguments and FVATTN_ELAUNCH if the HIP
 * runtime query fails (for instance with no GPU).
 */
int fvattn_attn_workers(int dtype, int d, int block, int v_layout, int group,
                        int* workers);

#ifdef __cplusplus
}
#endif

#endif /* FVATTN_H */
