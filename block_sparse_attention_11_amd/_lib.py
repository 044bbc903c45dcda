"""ctypes binding of libfvattn.so.

Argument marshalling only: every function takes torch tensors (device memory
allocated by the caller), checks dtype / shape / contiguity, and passes raw
pointers plus torch's current HIP stream to the C entry point of the same
name.  All compute happens in the library's HIP kernels; if the library is
missing this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libfvattn.so")
HEADER = os.path.join(ROOT, "include", "fvattn.h")

OK, EINVAL, EUNSUPPORTED, ELAUNCH, EWORKSPACE, ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 8 << 20
F32, BF16 = 0, 1
SCHED_TILE_ORDER = 1


def SCHED_GROUPS(x: int) -> int:
    """fvattn_schedule flag for the two-level LPT over x worker groups."""
    return int(x) << 8
V_ROWS, V_TILES = 0, 1

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_size_t = ctypes.c_size_t
_c_double = ctypes.c_double

_SIGNATURES = {
    "fvattn_status_string": (ctypes.c_char_p, [_c_int]),
    "fvattn_version": (_c_int, []),
    "fvattn_hilbert_permute": (_c_int, [_c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                        _c_void_p]),
    "fvattn_permute_rows": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                     _c_int, _c_int, _c_void_p]),
    "fvattn_pack_v": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int,
                               _c_int, _c_int, _c_void_p]),
    "fvattn_route_workspace_size": (_c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    "fvattn_route": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                              _c_int, _c_float, _c_int, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                              _c_void_p]),
    "fvattn_permute_pool": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                     _c_int, _c_int, _c_int, _c_void_p, _c_void_p]),
    "fvattn_route_pooled": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                     _c_float, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                     _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "fvattn_schedule_workspace_size": (_c_size_t, [_c_int, _c_int, _c_int]),
    "fvattn_schedule": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_void_p,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_size_t, _c_void_p]),
    "fvattn_schedule_noalloc": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p]),
    "fvattn_attn_workers": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                                     ctypes.POINTER(_c_int)]),
    "fvattn_sparse_attn": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_float, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _c_int, _c_void_p, _c_void_p, _c_int,
                                    _c_void_p, _c_void_p]),
    "fvattn_schedule_heads": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "fvattn_sasa_plan": (_c_int, [_c_void_p, _c_int, _c_int, _c_double, _c_double,
                                  _c_double, _c_double, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p]),
    "fvattn_sasa_workspace_size": (_c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    "fvattn_sasa_augment": (_c_int, [_c_void_p, _c_size_t, _c_int, _c_int, _c_int, _c_int,
                                     _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                     _c_size_t, _c_void_p]),
}


class FvattnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the in-tree libfvattn.so (built by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def declared_symbols() -> list:
    """Entry points declared in include/fvattn.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^;(]*?\b(fvattn_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return load_library().fvattn_status_string(status).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise FvattnError(fn, status, status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t=None):
    dev = t.device if t is not None else torch.device("cuda", torch.cuda.current_device())
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous on the GPU")


def hilbert_permute(T: int, Y: int, X: int, perm: torch.Tensor, inv_perm: torch.Tensor):
    _dev(perm, inv_perm)
    _need(perm.dtype == torch.int32 and inv_perm.dtype == torch.int32, "int32 outputs")
    _need(perm.numel() == T * Y * X == inv_perm.numel(), "outputs must hold T*Y*X")
    _check("fvattn_hilbert_permute", load_library().fvattn_hilbert_permute(
        T, Y, X, _ptr(perm), _ptr(inv_perm), _stream(perm)))


def permute_rows(src: torch.Tensor, dst: torch.Tensor, index: torch.Tensor):
    _dev(src, dst, index)
    _need(src.dim() == 3 and src.shape == dst.shape and src.dtype == dst.dtype,
          "src/dst must be [heads, n, d] of one dtype")
    _need(index.dtype == torch.int32 and index.numel() == src.shape[1], "index int32[n]")
    H, n, d = src.shape
    _check("fvattn_permute_rows", load_library().fvattn_permute_rows(
        _ptr(src), _ptr(dst), _ptr(index), H, n, d, _dtype_code(src), _stream(src)))


def pack_v(src: torch.Tensor, dst: torch.Tensor, index: torch.Tensor, block: int):
    """dst [heads, nB, d, block] <- rows of src [heads, n, d] gathered by index,
    one transposed tile per key block (padding keys zero)."""
    _dev(src, dst, index)
    _need(src.dim() == 3 and src.dtype == dst.dtype, "src [heads, n, d]")
    H, n, d = src.shape
    nb = (n + block - 1) // block
    _need(dst.numel() == H * nb * d * block, "dst must hold heads*nB*d*block")
    _need(index.dtype == torch.int32 and index.numel() == n, "index int32[n]")
    _check("fvattn_pack_v", load_library().fvattn_pack_v(
        _ptr(src), _ptr(dst), _ptr(index), H, n, d, block, _dtype_code(src), _stream(src)))


def route_workspace_size(heads: int, n: int, d: int, block: int) -> int:
    return int(load_library().fvattn_route_workspace_size(heads, n, d, block))


def route(q, k, block: int, p: float, k_floor: int, mask, kv_count, kv_index,
          head_load, head_density, workspace):
    _dev(q, k, mask, kv_count, kv_index, head_load, head_density, workspace)
    _need(q.shape == k.shape and q.dim() == 3 and q.dtype == k.dtype, "q, k [H, n, d]")
    H, n, d = q.shape
    nb = (n + block - 1) // block
    _need(mask.dtype == torch.uint8 and mask.numel() == H * nb * nb, "mask u8[H,nB,nB]")
    _need(kv_count.dtype == torch.int32 and kv_count.numel() == H * nb, "kv_count")
    _need(kv_index.dtype == torch.int32 and kv_index.numel() == H * nb * nb, "kv_index")
    _need(head_load.dtype == torch.int64 and head_load.numel() == H, "head_load")
    _need(head_density.dtype == torch.float32 and head_density.numel() == H,
          "head_density")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("fvattn_route", load_library().fvattn_route(
        _ptr(q), _ptr(k), _dtype_code(q), H, n, d, block, float(p), int(k_floor),
        _ptr(mask), _ptr(kv_count), _ptr(kv_index), _ptr(head_load),
        _ptr(head_density), _ptr(workspace), ws_bytes, _stream(q)))


def permute_pool(src: torch.Tensor, dst: torch.Tensor, index: torch.Tensor, block: int,
                 pooled: torch.Tensor):
    """dst <- rows of src gathered by index, and pooled [heads, nB, d] fp32 <-
    the column means of each block of dst rows, in one pass."""
    _dev(src, dst, index, pooled)
    _need(src.dim() == 3 and src.shape == dst.shape and src.dtype == dst.dtype,
          "src/dst must be [heads, n, d] of one dtype")
    H, n, d = src.shape
    nb = (n + block - 1) // block
    _need(index.dtype == torch.int32 and index.numel() == n, "index int32[n]")
    _need(pooled.dtype == torch.float32 and pooled.numel() == H * nb * d,
          "pooled f32[heads, nB, d]")
    _check("fvattn_permute_pool", load_library().fvattn_permute_pool(
        _ptr(src), _ptr(dst), _ptr(index), H, n, d, block, _dtype_code(src), _ptr(pooled),
        _stream(src)))


def route_pooled(qbar, kbar, n: int, block: int, p: float, k_floor: int, mask, kv_count,
                 kv_index, head_load, head_density, workspace):
    """route() from pooled means qbar, kbar [heads, nB, d] fp32 of n-row tensors."""
    _dev(qbar, kbar, mask, kv_count, kv_index, head_load, head_density, workspace)
    _need(qbar.shape == kbar.shape and qbar.dim() == 3 and qbar.dtype == torch.float32
          and kbar.dtype == torch.float32, "qbar, kbar f32[H, nB, d]")
    H, nb, d = qbar.shape
    _need(nb == (n + block - 1) // block, "qbar rows must be ceil(n / block)")
    _need(mask.dtype == torch.uint8 and mask.numel() == H * nb * nb, "mask u8[H,nB,nB]")
    _need(kv_count.dtype == torch.int32 and kv_count.numel() == H * nb, "kv_count")
    _need(kv_index.dtype == torch.int32 and kv_index.numel() == H * nb * nb, "kv_index")
    _need(head_load.dtype == torch.int64 and head_load.numel() == H, "head_load")
    _need(head_density.dtype == torch.float32 and head_density.numel() == H,
          "head_density")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("fvattn_route_pooled", load_library().fvattn_route_pooled(
        _ptr(qbar), _ptr(kbar), H, n, d, block, float(p), int(k_floor),
        _ptr(mask), _ptr(kv_count), _ptr(kv_index), _ptr(head_load),
        _ptr(head_density), _ptr(workspace), ws_bytes, _stream(qbar)))


def schedule_workspace_size(heads: int, n_qblocks: int, n_workers: int) -> int:
    return int(load_library().fvattn_schedule_workspace_size(heads, n_qblocks, n_workers))


def schedule(kv_count, n_workers: int, lpt_order, worker_offsets, worker_tiles,
             worker_load, workspace, tile_order: bool = False, group: int = 1,
             worker_groups: int = 1):
    """LPT lists over tiles of `group` q-blocks (tiles = H * ceil(nB / group));
    worker_groups > 1 selects the two-level LPT (heads to groups w % x)."""
    _dev(kv_count, lpt_order, worker_offsets, worker_tiles, worker_load, workspace)
    _need(kv_count.dim() == 2 and kv_count.dtype == torch.int32, "kv_count i32[H, nB]")
    H, nb = kv_count.shape
    tiles = H * ((nb + group - 1) // group)
    _need(lpt_order.numel() == tiles and worker_tiles.numel() == tiles, "tile arrays")
    _need(worker_offsets.numel() == n_workers + 1, "worker_offsets[W+1]")
    _need(worker_load.numel() == n_workers and worker_load.dtype == torch.int64,
          "worker_load i64[W]")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("fvattn_schedule", load_library().fvattn_schedule(
        _ptr(kv_count), H, nb, int(group), int(n_workers),
        (SCHED_TILE_ORDER if tile_order else 0)
        | (SCHED_GROUPS(worker_groups) if worker_groups > 1 else 0),
        _ptr(lpt_order), _ptr(worker_offsets),
        _ptr(worker_tiles), _ptr(worker_load), _ptr(workspace), ws_bytes,
        _stream(kv_count)))


def schedule_noalloc(kv_count, n_workers: int, lpt_order, worker_offsets, worker_tiles,
                     worker_load, tile_order: bool = False, group: int = 1,
                     worker_groups: int = 1):
    """schedule() with the library's static device scratch instead of a
    workspace (for callers that cannot allocate); same outputs."""
    _dev(kv_count, lpt_order, worker_offsets, worker_tiles, worker_load)
    _need(kv_count.dim() == 2 and kv_count.dtype == torch.int32, "kv_count i32[H, nB]")
    H, nb = kv_count.shape
    tiles = H * ((nb + group - 1) // group)
    _need(lpt_order.numel() == tiles and worker_tiles.numel() == tiles, "tile arrays")
    _need(worker_offsets.numel() == n_workers + 1, "worker_offsets[W+1]")
    _need(worker_load.numel() == n_workers and worker_load.dtype == torch.int64,
          "worker_load i64[W]")
    _check("fvattn_schedule_noalloc", load_library().fvattn_schedule_noalloc(
        _ptr(kv_count), H, nb, int(group), int(n_workers),
        (SCHED_TILE_ORDER if tile_order else 0)
        | (SCHED_GROUPS(worker_groups) if worker_groups > 1 else 0),
        _ptr(lpt_order), _ptr(worker_offsets),
        _ptr(worker_tiles), _ptr(worker_load), _stream(kv_count)))


def sparse_attn(q, k, v, o, block: int, kv_count, kv_index, worker_offsets=None,
                worker_tiles=None, n_workers: int = 0, timing=None, scale: float = 0.0,
                v_tiles: bool = False, group: int = 1, claims=None, out_rows=None,
                claim_groups: int = 0):
    """v is [H, n, d] (v_tiles=False) or [H, nB, d, block] tiles (v_tiles=True).
    claims: optional int32 [n_workers] scratch that turns on run-time
    balancing of the persistent launch (reset by the call); claim_groups > 1
    keeps every claim inside the workgroup's own group w % claim_groups.
    out_rows: optional int32 [n]; result row r goes to row out_rows[r] of o."""
    _dev(q, k, v, o, kv_count, kv_index)
    _need(q.shape == k.shape == o.shape and q.dim() == 3, "q,k,o [H, n, d]")
    _need(q.dtype == k.dtype == v.dtype == o.dtype, "one dtype")
    H, n, d = q.shape
    nb = (n + block - 1) // block
    if v_tiles:
        _need(v.numel() == H * nb * d * block, "v tiles [H, nB, d, block]")
    else:
        _need(v.shape == q.shape, "v [H, n, d]")
    _need(kv_count.numel() == H * nb and kv_index.numel() == H * nb * nb, "kv lists")
    if worker_offsets is not None:
        _dev(worker_offsets, worker_tiles)
        _need(worker_offsets.numel() == n_workers + 1, "worker_offsets[W+1]")
    if timing is not None:
        _dev(timing)
        _need(timing.numel() == 4 * n_workers and timing.element_size() == 8,
              "timing u64[W][4]")
    if out_rows is not None:
        _dev(out_rows)
        _need(out_rows.numel() == n and out_rows.dtype == torch.int32, "out_rows i32[n]")
    if claims is not None:
        _dev(claims)
        _need(claims.numel() == n_workers and claims.dtype == torch.int32, "claims i32[W]")
    _check("fvattn_sparse_attn", load_library().fvattn_sparse_attn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(q), H, n, d, block,
        V_TILES if v_tiles else V_ROWS, int(group), float(scale), _ptr(kv_count),
        _ptr(kv_index), _ptr(worker_offsets), _ptr(worker_tiles), int(n_workers),
        _ptr(timing), _ptr(claims), int(claim_groups), _ptr(out_rows), _stream(q)))


def schedule_heads(kv_count, n_workers: int, head_group, n_groups: int, lpt_order,
                   worker_offsets, worker_tiles, worker_load, workspace,
                   tile_order: bool = False, group: int = 1):
    """Two-level LPT with the head -> group map given (int32 [H])."""
    _dev(kv_count, head_group, lpt_order, worker_offsets, worker_tiles, worker_load,
         workspace)
    _need(kv_count.dim() == 2 and kv_count.dtype == torch.int32, "kv_count i32[H, nB]")
    H, nb = kv_count.shape
    tiles = H * ((nb + group - 1) // group)
    _need(head_group.numel() == H and head_group.dtype == torch.int32, "head_group i32[H]")
    _need(lpt_order.numel() == tiles and worker_tiles.numel() == tiles, "tile arrays")
    _need(worker_offsets.numel() == n_workers + 1, "worker_offsets[W+1]")
    _need(worker_load.numel() == n_workers and worker_load.dtype == torch.int64,
          "worker_load i64[W]")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("fvattn_schedule_heads", load_library().fvattn_schedule_heads(
        _ptr(kv_count), H, nb, int(group), int(n_workers), int(n_groups), _ptr(head_group),
        SCHED_TILE_ORDER if tile_order else 0, _ptr(lpt_order), _ptr(worker_offsets),
        _ptr(worker_tiles), _ptr(worker_load), _ptr(workspace), ws_bytes,
        _stream(kv_count)))


# the pages' SASA / RLB constants
SASA_K1, SASA_K2, SASA_N1, SASA_N2 = 1.05, 1.10, 0.8, 0.07


def sasa_plan(head_load, n_groups: int, head_group, group_budget, info,
              k1: float = SASA_K1, k2: float = SASA_K2, n1: float = SASA_N1,
              n2: float = SASA_N2):
    """Mode, head moves and per-group budgets (device outputs)."""
    _dev(head_load, head_group, group_budget, info)
    H = head_load.numel()
    _need(head_load.dtype == torch.int64, "head_load i64[H]")
    _need(head_group.numel() == H and head_group.dtype == torch.int32, "head_group i32[H]")
    _need(group_budget.numel() == n_groups and group_budget.dtype == torch.int64,
          "group_budget i64[G]")
    _need(info.numel() == 2 + 2 * n_groups and info.dtype == torch.int64, "info i64[2+2G]")
    _check("fvattn_sasa_plan", load_library().fvattn_sasa_plan(
        _ptr(head_load), H, int(n_groups), float(k1), float(k2), float(n1), float(n2),
        _ptr(head_group), _ptr(group_budget), _ptr(info), _stream(head_load)))


def sasa_workspace_size(heads: int, n: int, block: int, n_groups: int) -> int:
    return int(load_library().fvattn_sasa_workspace_size(heads, n, block, n_groups))


def sasa_augment(route_workspace, heads: int, n: int, d: int, block: int, head_group,
                 group_budget, mask, kv_count, kv_index, head_load, head_density, added,
                 workspace):
    """Adds each group's budget of skipped blocks, most important first, and
    rewrites the routing outputs (route_workspace: that of the route call)."""
    _dev(route_workspace, head_group, group_budget, mask, kv_count, kv_index, head_load,
         head_density, added, workspace)
    G = group_budget.numel()
    nb = (n + block - 1) // block
    _need(mask.dtype == torch.uint8 and mask.numel() == heads * nb * nb, "mask u8[H,nB,nB]")
    _need(kv_count.dtype == torch.int32 and kv_count.numel() == heads * nb, "kv_count")
    _need(kv_index.dtype == torch.int32 and kv_index.numel() == heads * nb * nb, "kv_index")
    _need(head_group.numel() == heads and head_group.dtype == torch.int32, "head_group")
    _need(group_budget.dtype == torch.int64 and added.dtype == torch.int64 and
          added.numel() == G, "budget / added i64[G]")
    _check("fvattn_sasa_augment", load_library().fvattn_sasa_augment(
        _ptr(route_workspace), route_workspace.numel() * route_workspace.element_size(),
        int(heads), int(n), int(d), int(block), _ptr(head_group), _ptr(group_budget), G,
        _ptr(mask), _ptr(kv_count), _ptr(kv_index), _ptr(head_load), _ptr(head_density),
        _ptr(added), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(mask)))


def attn_workers(dtype: torch.dtype, d: int, block: int, v_tiles: bool,
                 group: int = 1) -> int:
    """Resident workgroups of the attention kernel on the current device."""
    out = _c_int(0)
    code = F32 if dtype == torch.float32 else BF16
    _check("fvattn_attn_workers", load_library().fvattn_attn_workers(
        code, d, block, V_TILES if v_tiles else V_ROWS, int(group), ctypes.byref(out)))
    return int(out.value)
