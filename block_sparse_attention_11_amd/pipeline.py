"""The whole hot path for one grid shape, with its buffers.

Allocation and call order only; each step is one C-ABI call into the HIP
library:

    hilbert_permute  (once per grid shape)
    permute_pool     Q, K -> Hilbert order, with the pooled block means in the
                     same pass (fused=False: permute_rows, pooling in route)
    pack_v           V -> Hilbert order, one transposed tile per key block; with
                     overlap=True on a second stream, started once routing is
                     queued so it runs beside the schedule (a few latency-bound
                     workgroups; V feeds neither), joined before attention
    route_pooled     pooled-Q/K Top-p + Top-k -> mask, kept lists, head load
    [sasa_plan, sasa_augment   per-rank image only: head moves and extra
                     blocks on the groups off the critical path]
    schedule         LPT work list over (head, q-block) tiles
    sparse_attn      persistent block-sparse attention over the kept blocks,
                     storing O straight back in token order

With ranks = G > 1 the path runs the per-rank image of the pages' system:
the persistent workers form G groups (worker w in group w % G; G = 8 puts
one group on each XCD), heads start in contiguous shards, the SASA plan may
move heads between groups (RLB) and, with sasa=True, adds each group's
budget of skipped high-importance blocks; every group then claims work only
from its own lists, so the groups finish independently, like ranks.
"""
from __future__ import annotations

import torch

from . import _lib

MAX_WORKERS = 2048          # fvattn_schedule's limit
XCDS = 8                    # accelerator complex dies of an MI355X


def default_workers(device=None) -> int:
    """Compute units of the device."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    return torch.cuda.get_device_properties(dev).multi_processor_count


class FVAttnPath:
    def __init__(self, heads: int, grid, d: int, block: int, dtype=torch.bfloat16,
                 n_workers: int | None = None, device="cuda", tile_order: bool = False,
                 v_tiles: bool | None = None, group: int | None = None,
                 worker_groups: int | None = None, ranks: int = 0, sasa: bool = False,
                 fused: bool = True, overlap: bool = True,
                 sasa_n1: float = _lib.SASA_N1):
        self.heads, self.grid, self.d, self.block = heads, tuple(grid), d, block
        T, Y, X = self.grid
        self.n = T * Y * X
        self.nb = (self.n + block - 1) // block
        self.dtype = dtype
        self.tile_order = tile_order
        # two-level LPT over the XCDs: persistent workgroup w runs on XCD
        # w % 8 of an MI355X, so 8 groups keep each head on one XCD (used when
        # there are at least two heads per group)
        self.device = torch.device(device)
        H, n, nb, dev = heads, self.n, self.nb, self.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.perm = torch.empty(n, **i32)
        self.inv_perm = torch.empty(n, **i32)
        # V goes to transposed key-block tiles when the bf16 tile packer applies
        can_tile = dtype == torch.bfloat16 and d % 8 == 0 and block % 16 == 0
        self.v_tiles = can_tile if v_tiles is None else (v_tiles and can_tile)
        self.qh = torch.empty((H, n, d), dtype=dtype, device=dev)
        self.kh = torch.empty_like(self.qh)
        self._vh = (torch.empty((H, nb, d, block), dtype=dtype, device=dev) if self.v_tiles
                    else torch.empty_like(self.qh))
        self.oh = torch.empty_like(self.qh)
        # tiles of two (or three) q-blocks share each K/V block load (tiled V only)
        self.group = (2 if self.v_tiles else 1) if group is None else group
        self.tiles = H * ((nb + self.group - 1) // self.group)
        with torch.cuda.device(dev):
            self.n_workers = n_workers or min(
                MAX_WORKERS, _lib.attn_workers(dtype, d, block, self.v_tiles, self.group))
        self.mask = torch.empty((H, nb, nb), dtype=torch.uint8, device=dev)
        self.kv_count = torch.empty((H, nb), **i32)
        self.kv_index = torch.empty((H, nb, nb), **i32)
        self.head_load = torch.empty(H, dtype=torch.int64, device=dev)
        self.head_density = torch.empty(H, dtype=torch.float32, device=dev)
        self.route_ws = torch.empty(_lib.route_workspace_size(H, n, d, block),
                                    dtype=torch.uint8, device=dev)
        # pooled block means, written by the Q/K gather when fused
        self.fused = fused
        if fused:
            self.qbar = torch.empty((H, nb, d), dtype=torch.float32, device=dev)
            self.kbar = torch.empty_like(self.qbar)
        # V layout on a side stream (default priority), joined before attention
        self.overlap = overlap
        self.side = torch.cuda.Stream(device=dev) if overlap else None
        self._v_pending = False
        self._v_src = None
        W = self.n_workers
        if worker_groups is None:
            # at least two heads per group, or the head-level LPT cannot balance
            worker_groups = XCDS if (W % XCDS == 0 and 2 * XCDS <= heads <= 4096) else 1
        self.worker_groups = worker_groups
        self.lpt_order = torch.empty(self.tiles, **i32)
        self.worker_offsets = torch.empty(W + 1, **i32)
        self.worker_tiles = torch.empty(self.tiles, **i32)
        self.worker_load = torch.empty(W, dtype=torch.int64, device=dev)
        self.sched_ws = torch.empty(_lib.schedule_workspace_size(H, nb, W),
                                    dtype=torch.uint8, device=dev)
        self.timing = torch.zeros((W, 4), dtype=torch.int64, device=dev)
        # claim counters for run-time balancing of the persistent launch
        self.claims = torch.zeros(W, dtype=torch.int32, device=dev)
        # per-rank image (SASA / RLB on the worker groups)
        if sasa and ranks < 2:
            raise ValueError("sasa needs ranks >= 2 (the per-rank image)")
        if ranks > 1 and (ranks > min(64, W) or W % ranks != 0):
            raise ValueError("ranks must divide the worker count and be <= 64")
        self.ranks, self.sasa = ranks, sasa
        # SASA's augmentation coefficient (the pages' n1 = 0.8 by default)
        self.sasa_n1 = sasa_n1
        if ranks > 1:
            i64 = dict(dtype=torch.int64, device=dev)
            self.head_group = torch.empty(H, **i32)
            self.group_budget = torch.empty(ranks, **i64)
            self.sasa_info = torch.empty(2 + 2 * ranks, **i64)
            self.sasa_added = torch.zeros(ranks, **i64)
            self.sasa_ws = torch.empty(_lib.sasa_workspace_size(H, n, block, ranks),
                                       dtype=torch.uint8, device=dev)
        self.ordered = False

    # -- steps -------------------------------------------------------------
    def order(self):
        _lib.hilbert_permute(*self.grid, self.perm, self.inv_perm)
        self.ordered = True

    def to_hilbert(self, q, k, v):
        if self.fused:
            _lib.permute_pool(q, self.qh, self.perm, self.block, self.qbar)
            _lib.permute_pool(k, self.kh, self.perm, self.block, self.kbar)
        else:
            _lib.permute_rows(q, self.qh, self.perm)
            _lib.permute_rows(k, self.kh, self.perm)
        if not self.overlap:
            self._layout_v(v)
            return
        # with overlap the V layout starts after routing is queued (start_v)
        self._v_src = v

    def start_v(self):
        """Queue the pending V layout on the side stream.  The side stream
        first waits for all work queued so far on the main one (v is ready,
        the previous attention has finished reading vh, routing is queued, so
        the layout shares the card with the schedule rather than with the
        bandwidth-heavy routing)."""
        v = self._v_src
        if v is None:
            return
        self._v_src = None
        main = torch.cuda.current_stream(self.device)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            self._layout_v(v)
        if not torch.cuda.is_current_stream_capturing():
            # keep v's memory for the side stream's read (a captured graph
            # holds its inputs itself)
            v.record_stream(self.side)
        self._v_pending = True

    def _layout_v(self, v):
        if self.v_tiles:
            _lib.pack_v(v, self._vh, self.perm, self.block)
        else:
            _lib.permute_rows(v, self._vh, self.perm)

    @property
    def vh(self):
        """V in Hilbert order; reading it first joins the side stream."""
        self.join()
        return self._vh

    def join(self):
        """Make the main stream wait for the V layout (no-op without overlap);
        a layout not yet started runs on the main stream."""
        if self._v_src is not None:
            v, self._v_src = self._v_src, None
            self._layout_v(v)
        if self._v_pending:
            torch.cuda.current_stream(self.device).wait_stream(self.side)
            self._v_pending = False

    def route(self, p: float, k_floor: int):
        if self.fused:
            _lib.route_pooled(self.qbar, self.kbar, self.n, self.block, p, k_floor, self.mask,
                              self.kv_count, self.kv_index, self.head_load,
                              self.head_density, self.route_ws)
        else:
            _lib.route(self.qh, self.kh, self.block, p, k_floor, self.mask, self.kv_count,
                       self.kv_index, self.head_load, self.head_density, self.route_ws)
        self.start_v()

    def plan_ranks(self):
        """Per-rank image: mode, head moves and budgets; with sasa, the extra
        blocks (rewrites mask, kv lists, head load and density)."""
        _lib.sasa_plan(self.head_load, self.ranks, self.head_group, self.group_budget,
                       self.sasa_info, n1=self.sasa_n1)
        if self.sasa:
            _lib.sasa_augment(self.route_ws, self.heads, self.n, self.d, self.block,
                              self.head_group, self.group_budget, self.mask, self.kv_count,
                              self.kv_index, self.head_load, self.head_density,
                              self.sasa_added, self.sasa_ws)

    def schedule(self):
        if self.ranks > 1:
            _lib.schedule_heads(self.kv_count, self.n_workers, self.head_group, self.ranks,
                                self.lpt_order, self.worker_offsets, self.worker_tiles,
                                self.worker_load, self.sched_ws,
                                tile_order=self.tile_order, group=self.group)
            return
        _lib.schedule(self.kv_count, self.n_workers, self.lpt_order, self.worker_offsets,
                      self.worker_tiles, self.worker_load, self.sched_ws,
                      tile_order=self.tile_order, group=self.group,
                      worker_groups=self.worker_groups)

    def attend(self, balanced: bool = True, timing: bool = True, runtime: bool = True,
               out=None):
        """balanced: persistent launch over the LPT lists (else the head-major
        grid control); runtime: with run-time claims on top of the lists.
        out: write O straight into `out` in token order (the kernels scatter
        rows through the Hilbert order); None: O stays in Hilbert order in
        self.oh."""
        self.join()
        o = self.oh if out is None else out
        rows = None if out is None else self.perm
        if balanced:
            _lib.sparse_attn(self.qh, self.kh, self.vh, o, self.block,
                             self.kv_count, self.kv_index, self.worker_offsets,
                             self.worker_tiles, self.n_workers,
                             self.timing if timing else None, v_tiles=self.v_tiles,
                             group=self.group, claims=self.claims if runtime else None,
                             out_rows=rows,
                             claim_groups=self.ranks if self.ranks > 1 else 0)
        else:
            _lib.sparse_attn(self.qh, self.kh, self.vh, o, self.block,
                             self.kv_count, self.kv_index, v_tiles=self.v_tiles,
                             group=self.group, out_rows=rows)

    def to_tokens(self, out):
        _lib.permute_rows(self.oh, out, self.inv_perm)

    def run(self, q, k, v, p: float, k_floor: int, out=None, balanced: bool = True,
            runtime: bool = True):
        """One pass of the whole path; returns O in token order."""
        if out is None:
            out = torch.empty_like(q)
        if not self.ordered:
            self.order()
        self.to_hilbert(q, k, v)
        self.route(p, k_floor)
        if self.ranks > 1:
            self.plan_ranks()
        self.schedule()
        self.attend(balanced, runtime=runtime, out=out)
        return out
