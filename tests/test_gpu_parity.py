"""GPU parity: every step of the HIP path against the CPU oracle, through the
C ABI, on seeded synthetic inputs.

Stage-wise on identical inputs: the oracle's LPT runs on the GPU's kv_count
and the oracle's attention on the GPU's kept lists; Hilbert order and LPT
must match bit for bit, masks per the row protocol in tests/parity.py, and
attention within max-abs 2e-2 (bf16) / 1e-4 (fp32) plus a relative-L2 bound.
"""

import numpy as np
import pytest
import torch

from block_sparse_attention_11_amd import _lib, synth
from block_sparse_attention_11_amd.pipeline import FVAttnPath
from oracle import attention as oat
from oracle import hilbert as ohb
from oracle import lpt as olpt
from oracle import route as ort
from tests.parity import TOL, attn_errors, classify_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def to_np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------------------
# Hilbert
# ---------------------------------------------------------------------------
GRIDS = [(1, 1, 1), (1, 1, 5), (2, 2, 2), (2, 8, 8), (3, 5, 7), (17, 1, 3),
         (4, 16, 16), (16, 16, 16), (21, 30, 52), (21, 45, 80), (41, 45, 80),
         (1, 300, 2), (33, 17, 65),
         # sides up to the largest the ABI takes (1024: 10 bits per axis)
         (1024, 1, 1), (1, 1, 1024), (3, 1024, 7), (1, 1024, 1024), (1024, 1024, 1),
         (513, 1000, 3)]


@pytest.mark.parametrize("grid", GRIDS)
def test_hilbert_bit_exact(grid):
    say(f"hilbert {grid}")
    n = grid[0] * grid[1] * grid[2]
    perm = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    inv = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    _lib.hilbert_permute(*grid, perm, inv)
    torch.cuda.synchronize()
    rp, ri = ohb.hilbert_order(*grid)
    assert np.array_equal(perm.cpu().numpy(), rp)
    assert np.array_equal(inv.cpu().numpy(), ri)


# ---------------------------------------------------------------------------
# Permute
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64),
                                     (torch.bfloat16, 6), (torch.float32, 3)])
def test_permute_rows_bit_exact(dtype, d):
    say(f"permute {dtype} d={d}")
    g = torch.Generator().manual_seed(5)
    H, n = 3, 1000
    x = torch.randn((H, n, d), generator=g).to(dtype)
    idx = torch.randperm(n, generator=g).to(torch.int32)
    dst = torch.empty((H, n, d), dtype=dtype, device=DEV)
    _lib.permute_rows(x.to(DEV), dst, idx.to(DEV))
    ref = ort.permute_rows(x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)
                           .numpy(), idx.numpy())
    got = dst.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("d,block,n", [(128, 128, 75600 // 40), (64, 64, 390), (64, 16, 105),
                                       (128, 64, 1000), (8, 16, 9), (16, 48, 50)])
def test_pack_v_bit_exact(d, block, n):
    say(f"pack_v d={d} block={block} n={n}")
    g = torch.Generator().manual_seed(11)
    H = 3
    x = torch.randn((H, n, d), generator=g).to(torch.bfloat16)
    idx = torch.randperm(n, generator=g).to(torch.int32)
    nb = (n + block - 1) // block
    dst = torch.full((H, nb, d, block), 7.0, dtype=torch.bfloat16, device=DEV)
    _lib.pack_v(x.to(DEV), dst, idx.to(DEV), block)
    torch.cuda.synchronize()
    xs = ort.permute_rows(x.view(torch.int16).numpy(), idx.numpy())      # [H, n, d]
    pad = np.zeros((H, nb * block, d), dtype=np.int16)
    pad[:, :n] = xs
    ref = pad.reshape(H, nb, block, d).transpose(0, 1, 3, 2)          # [H, nb, d, block]
    # inside each 16-key group of a tile row the 4-key units are stored in
    # the order 0, 2, 1, 3
    groups = ref.reshape(H, nb, d, block // 16, 4, 4)
    want = groups[:, :, :, :, [0, 2, 1, 3], :]
    assert np.array_equal(dst.cpu().view(torch.int16).numpy(),
                          want.reshape(H, nb, d, block))


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------
def run_route(w, q, k, p, kf, fused=True):
    """GPU gather + route; fused: pooling in the gather (permute_pool +
    route_pooled), else permute_rows + route."""
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, n_workers=8, device=DEV,
                      fused=fused)
    path.order()
    path.to_hilbert(q, k, k)
    path.route(p, kf)
    torch.cuda.synchronize()
    return path


ROUTE_CASES = [
    ("tiny", None, None),
    ("small", None, None),
    ("small", 0.5, 1),
    ("small", 1.0, 0),
    ("small", 0.2, 20),      # floor beyond nB
    ("ragged_f32", 0.6, 2),
    ("ragged_bf16", 0.8, 3),
    ("mid_bf16", 0.95, 8),
]


def workload(name):
    W = synth.WORKLOADS
    if name in W:
        return W[name]
    if name == "ragged_f32":
        return synth.Workload("ragged_f32", 2, 32, (3, 5, 7), 16, 0.6, 2, "f32")
    if name == "ragged_bf16":
        return synth.Workload("ragged_bf16", 3, 64, (3, 5, 7), 16, 0.8, 3, "bf16",
                              s_range=(1.0, 64.0))
    if name == "mid_bf16":
        # several 128-blocks with an 80-row tail, MFMA shape (d=128, block=128)
        return synth.Workload("mid_bf16", 3, 128, (5, 9, 16), 128, 0.95, 8, "bf16",
                              s_range=(4.0, 256.0))
    if name == "mid_bf16_64":
        return synth.Workload("mid_bf16_64", 2, 64, (3, 10, 13), 64, 0.9, 4, "bf16",
                              s_range=(2.0, 128.0))
    if name == "mid8_bf16":
        # 8 blocks of 128 (4-row tail): tiles of three q-blocks end in a pair
        return synth.Workload("mid8_bf16", 3, 128, (5, 9, 20), 128, 0.9, 4, "bf16",
                              s_range=(4.0, 256.0))
    if name == "mid7_bf16_64":
        # d = 64, 7 blocks of 128 (102-row tail): the last tile of three holds one
        return synth.Workload("mid7_bf16_64", 2, 64, (3, 10, 29), 128, 0.9, 4, "bf16",
                              s_range=(2.0, 128.0))
    raise KeyError(name)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("name,p,kf", ROUTE_CASES)
def test_route_parity(name, p, kf, fused):
    w = workload(name)
    p = w.p if p is None else p
    kf = w.k if kf is None else kf
    say(f"route {name} p={p} k={kf} fused={fused}")
    q, k, v, _ = synth.make_inputs(w, "cpu")
    path = run_route(w, q.to(DEV), k.to(DEV), p, kf, fused)
    perm, _ = ohb.hilbert_order(*w.grid)
    assert np.array_equal(path.perm.cpu().numpy(), perm)
    qh = ort.permute_rows(to_np(q).astype(np.float64), perm)
    kh = ort.permute_rows(to_np(k).astype(np.float64), perm)
    # the GPU's Hilbert-ordered copies are the same bytes
    assert np.array_equal(to_np(path.qh), qh.astype(to_np(path.qh).dtype))
    ora = ort.route(qh, kh, w.block, p, kf)
    assert np.array_equal(to_np(path.kh), kh.astype(to_np(path.kh).dtype))
    ws = path.route_ws
    nb, H, d = path.nb, w.heads, w.d
    if fused:
        qbar, kbar = path.qbar.cpu().numpy(), path.kbar.cpu().numpy()
    else:
        qbar = ws[:H * nb * d * 4].view(torch.float32).reshape(H, nb, d).cpu().numpy()
        kbar = None
    assert np.allclose(qbar, ora["qbar"], rtol=1e-5, atol=1e-6)
    if kbar is not None:
        assert np.allclose(kbar, ora["kbar"], rtol=1e-5, atol=1e-6)
    gc = path.kv_count.cpu().numpy()
    gi = path.kv_index.cpu().numpy()
    stats, bad = classify_rows(ora["P"], p, kf, gc, gi, ora["kv_count"], ora["kv_index"])
    say(f"  mask rows {stats}")
    assert stats["unexplained"] == 0, bad[:10]
    gm = path.mask.cpu().numpy()
    for h in range(H):
        for i in range(nb):
            assert np.flatnonzero(gm[h, i]).tolist() == gi[h, i, :gc[h, i]].tolist()
    load = path.head_load.cpu().numpy()
    assert np.array_equal(load, gc.astype(np.int64).sum(1))
    dens = path.head_density.cpu().numpy()
    assert np.array_equal(dens, (load / float(nb * nb)).astype(np.float32))
    assert (gc >= min(kf, nb)).all()


# ---------------------------------------------------------------------------
# LPT schedule
# ---------------------------------------------------------------------------
def gpu_schedule(costs_2d, W, tile_order=False, group=1, worker_groups=1):
    H, nb = costs_2d.shape
    kvc = torch.from_numpy(costs_2d.astype(np.int32)).to(DEV)
    tiles = H * ((nb + group - 1) // group)
    order = torch.empty(tiles, dtype=torch.int32, device=DEV)
    off = torch.empty(W + 1, dtype=torch.int32, device=DEV)
    wt = torch.empty(tiles, dtype=torch.int32, device=DEV)
    wl = torch.empty(W, dtype=torch.int64, device=DEV)
    ws = torch.empty(_lib.schedule_workspace_size(H, nb, W), dtype=torch.uint8, device=DEV)
    _lib.schedule(kvc, W, order, off, wt, wl, ws, tile_order=tile_order, group=group,
                  worker_groups=worker_groups)
    torch.cuda.synchronize()
    return order.cpu().numpy(), off.cpu().numpy(), wt.cpu().numpy(), wl.cpu().numpy()


SCHED_CASES = [
    ("hand", np.array([[7, 5, 4, 3, 3, 2]]), 2),
    ("one_worker", np.array([[4, 9, 1, 9, 0]]), 1),
    ("more_workers", np.array([[2, 5, 5]]), 5),
    ("all_zero", np.zeros((2, 7), dtype=np.int64), 3),
    ("equal", np.full((40, 591), 561), 256),
    ("random_ties", None, 64),
    ("random_wide", None, 1024),
    ("max_workers", None, 2048),
    ("random_odd", None, 100),
    ("big_costs", None, 256),
    ("max_heads", None, 256),        # the most heads the two-level schedule takes
    # every head's load passes 2^26: groups holding one leave the one-wavefront
    # assignment for the batch kernel, empty groups stay on the wavefront
    ("huge_loads", None, 256),
]


# worker-group counts per case: the two-level schedule needs two workers or
# more (with one worker it is the plain schedule, which xg = 1 covers)
SCHED_PARAMS = [(name, costs, W, xg) for name, costs, W in SCHED_CASES
                for xg in ([1, 8, 3] if W > 1 else [1])]


@pytest.mark.parametrize("group", [1, 2, 3])
@pytest.mark.parametrize("tile_order", [False, True])
@pytest.mark.parametrize("name,costs,W,xg", SCHED_PARAMS,
                         ids=[f"{p[0]}-W{p[2]}-x{p[3]}" for p in SCHED_PARAMS])
def test_schedule_bit_exact(name, costs, W, tile_order, group, xg):
    X = min(xg, W)
    say(f"schedule {name} W={W} tile_order={tile_order} group={group} groups={X}")
    rng = np.random.default_rng(sum(map(ord, name)))
    if name == "random_ties":
        costs = rng.integers(1, 9, size=(8, 37))
    elif name in ("random_wide", "max_workers"):
        costs = rng.integers(0, 600, size=(40, 591))
    elif name == "random_odd":
        costs = rng.integers(8, 1155, size=(40, 1154))
    elif name == "big_costs":
        costs = rng.integers(0, 16384, size=(5, 333))
    elif name == "max_heads":
        costs = rng.integers(0, 50, size=(4096, 3))
    elif name == "huge_loads":
        # tiles stay inside the 65535 cost clamp of the schedule ABI
        if group == 3:
            costs = rng.integers(21000, 21845, size=(3, 3300))
        else:
            costs = rng.integers(32000, 32768, size=(3, 2100))
        assert costs.sum(1).min() >= 2 ** 26
        assert olpt.group_costs(costs, group).max() <= 65535
    got = gpu_schedule(costs, W, tile_order, group, X)
    gc = olpt.group_costs(costs, group)
    if X > 1:
        ref = olpt.lpt_schedule_grouped(gc.reshape(costs.shape[0], -1), W, X,
                                        tile_order=tile_order)
    else:
        ref = olpt.lpt_schedule(gc, W, tile_order=tile_order)
    for g, r, what in zip(got, ref, ("order", "offsets", "tiles", "loads")):
        assert np.array_equal(g, r), what


# ---------------------------------------------------------------------------
# Attention on the GPU's kept lists
# ---------------------------------------------------------------------------
ATTN_CASES = ["tiny", "small", "ragged_f32", "ragged_bf16", "mid_bf16", "mid_bf16_64"]


@pytest.mark.parametrize("name", ATTN_CASES)
@pytest.mark.parametrize("balanced", [True, False])
@pytest.mark.parametrize("v_tiles,group", [(True, 2), (True, 1), (False, 1), (False, 2)])
def test_attention_parity(name, balanced, v_tiles, group):
    w = workload(name)
    say(f"attention {name} balanced={balanced} v_tiles={v_tiles} group={group}")
    q, k, v, _ = synth.make_inputs(w, "cpu")
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, n_workers=7,
                      device=DEV, v_tiles=v_tiles, group=group)
    out = path.run(q.to(DEV), k.to(DEV), v.to(DEV), w.p, w.k, balanced=balanced)
    torch.cuda.synchronize()
    perm = path.perm.cpu().numpy()
    qh, kh, vh = (ort.permute_rows(to_np(x).astype(np.float64), perm) for x in (q, k, v))
    ref_h = oat.block_sparse_attention(qh, kh, vh, w.block, path.kv_count.cpu().numpy(),
                                       path.kv_index.cpu().numpy())
    ref = oat.unpermute_rows(ref_h, perm)
    err = attn_errors(to_np(out), ref)
    say(f"  {err}")
    tol = TOL[w.dtype]
    assert err["max_abs"] <= tol["max_abs"] and err["rel_l2"] <= tol["rel_l2"], err
    # run() scatters O back to token order inside the attention kernel; the
    # same launch without the scatter leaves the same bits in Hilbert order
    path.attend(balanced)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(path.oh), ort.permute_rows(to_np(out), perm))


@pytest.mark.parametrize("name", ["mid_bf16", "mid8_bf16", "mid7_bf16_64"])
@pytest.mark.parametrize("balanced", [True, False])
def test_attention_parity_three_qblocks(name, balanced):
    """Tiles of three q-blocks (group 3, V tiles, 128-key blocks), with the
    last tile of a head holding three, two or one q-blocks."""
    w = workload(name)
    say(f"attention group 3 {name} balanced={balanced}")
    q, k, v, _ = synth.make_inputs(w, "cpu")
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, n_workers=5,
                      device=DEV, group=3)
    assert path.v_tiles and path.group == 3
    out = path.run(q.to(DEV), k.to(DEV), v.to(DEV), w.p, w.k, balanced=balanced)
    torch.cuda.synchronize()
    perm = path.perm.cpu().numpy()
    qh, kh, vh = (ort.permute_rows(to_np(x).astype(np.float64), perm) for x in (q, k, v))
    ref = oat.unpermute_rows(oat.block_sparse_attention(
        qh, kh, vh, w.block, path.kv_count.cpu().numpy(), path.kv_index.cpu().numpy()), perm)
    err = attn_errors(to_np(out), ref)
    say(f"  {err}")
    tol = TOL[w.dtype]
    assert err["max_abs"] <= tol["max_abs"] and err["rel_l2"] <= tol["rel_l2"], err
    if balanced:
        # the schedule of three-q-block tiles against the oracle
        gc = olpt.group_costs(path.kv_count.cpu().numpy(), 3)
        ref_s = olpt.lpt_schedule(gc, path.n_workers) if path.worker_groups == 1 else \
            olpt.lpt_schedule_grouped(gc.reshape(w.heads, -1), path.n_workers,
                                      path.worker_groups)
        for g, r in zip((path.lpt_order, path.worker_offsets, path.worker_tiles,
                         path.worker_load), ref_s):
            assert np.array_equal(g.cpu().numpy(), r)


@pytest.mark.parametrize("name", ["small", "mid_bf16", "ragged_f32"])
def test_dense_control_matches_brute_force(name):
    """p = 1 keeps every block: the path must equal plain dense attention in
    the original token order."""
    w = workload(name)
    say(f"dense control {name}")
    q, k, v, _ = synth.make_inputs(w, "cpu")
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, device=DEV)
    out = path.run(q.to(DEV), k.to(DEV), v.to(DEV), 1.0, 0)
    torch.cuda.synchronize()
    assert (path.kv_count.cpu().numpy() == path.nb).all()
    assert (path.head_density.cpu().numpy() == 1.0).all()
    ref = oat.dense_attention(to_np(q), to_np(k), to_np(v))
    err = attn_errors(to_np(out), ref)
    say(f"  {err}")
    tol = TOL[w.dtype]
    assert err["max_abs"] <= tol["max_abs"] and err["rel_l2"] <= tol["rel_l2"], err


def attn_call(q, k, v, o, block, cnt, idx, v_tiles, group=1, **kw):
    """sparse_attn with V given as rows or packed into tiles (identity order)."""
    if v_tiles:
        H, n, d = v.shape
        nb = (n + block - 1) // block
        vt = torch.empty((H, nb, d, block), dtype=v.dtype, device=DEV)
        _lib.pack_v(v, vt, torch.arange(n, dtype=torch.int32, device=DEV), block)
        v = vt
    _lib.sparse_attn(q, k, v, o, block, cnt, idx, v_tiles=v_tiles, group=group, **kw)


@pytest.mark.parametrize("dtype,d,block,v_tiles,group", [
    (torch.bfloat16, 128, 128, True, 2), (torch.bfloat16, 128, 128, True, 1),
    (torch.bfloat16, 128, 128, False, 1), (torch.bfloat16, 64, 64, True, 2),
    (torch.bfloat16, 64, 64, False, 2), (torch.bfloat16, 64, 16, True, 1),
    (torch.float32, 64, 16, False, 2), (torch.bfloat16, 128, 128, True, 3),
    (torch.bfloat16, 64, 128, True, 3)])
def test_attention_handmade_lists(dtype, d, block, v_tiles, group):
    """Edge cases: an empty row (written as zeros), a single kept block, only
    the short tail block, a pair whose two lists differ, and constant V."""
    say(f"handmade lists {dtype} d={d} block={block} v_tiles={v_tiles} group={group}")
    H, n = 2, 3 * block + block // 2 + 1
    nb = 4
    g = torch.Generator().manual_seed(3)
    q = (torch.randn((H, n, d), generator=g) * 2).to(dtype)
    k = (torch.randn((H, n, d), generator=g) * 2).to(dtype)
    v = torch.randn((H, n, d), generator=g).to(dtype)
    cnt = np.array([[0, 1, 1, 4], [2, 1, 3, 1]], dtype=np.int32)
    idx = np.zeros((H, nb, nb), dtype=np.int32)
    idx[0, 1, 0] = 3
    idx[0, 2, 0] = 0
    idx[0, 3, :4] = [0, 1, 2, 3]
    idx[1, 0, :2] = [1, 3]
    idx[1, 1, 0] = 1
    idx[1, 2, :3] = [0, 2, 3]
    idx[1, 3, 0] = 3
    o = torch.full((H, n, d), float("nan"), dtype=dtype, device=DEV)
    attn_call(q.to(DEV), k.to(DEV), v.to(DEV), o, block,
              torch.from_numpy(cnt).to(DEV), torch.from_numpy(idx).to(DEV), v_tiles, group)
    torch.cuda.synchronize()
    got = to_np(o)
    qq, kk, vv = (to_np(x).astype(np.float64) for x in (q, k, v))
    assert (got[0, :block] == 0).all()
    tiles = [(h, i) for h in range(H) for i in range(nb) if cnt[h, i] > 0]
    ref = oat.block_sparse_attention(qq, kk, vv, block, cnt, idx, tiles=tiles)
    mask = ~np.isnan(ref)
    err = attn_errors(got[mask], ref[mask])
    tol = TOL["bf16" if dtype == torch.bfloat16 else "f32"]
    assert err["max_abs"] <= tol["max_abs"] and err["rel_l2"] <= tol["rel_l2"], err
    # constant V rows give the constant, whatever the mask
    vc = torch.arange(d, dtype=torch.float32).div(d).expand(H, n, d).contiguous().to(dtype)
    attn_call(q.to(DEV), k.to(DEV), vc.to(DEV), o, block,
              torch.from_numpy(cnt).to(DEV), torch.from_numpy(idx).to(DEV), v_tiles, group)
    torch.cuda.synchronize()
    got = to_np(o)
    exp = to_np(vc)
    for h, i in tiles:
        r0, r1 = i * block, min(n, (i + 1) * block)
        assert np.abs(got[h, r0:r1] - exp[h, r0:r1]).max() <= tol["max_abs"]


@pytest.mark.parametrize("layout", ["one_list", "round_robin", "reversed", "more_workers"])
@pytest.mark.parametrize("group", [2, 3])
def test_runtime_claims(layout, group):
    """Run-time balancing: with claim counters the workgroups take tiles from
    other workers' lists; every tile still runs once, in one workgroup, so the
    output equals the static-list run bit for bit.  Includes a tile with
    nothing kept (zeroed by the claiming workgroup)."""
    w = workload("mid_bf16" if group == 2 else "mid8_bf16")
    say(f"runtime claims {layout} group={group}")
    q, k, v, _ = synth.make_inputs(w, "cpu")
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, device=DEV, group=group)
    assert path.group == group and path.v_tiles
    path.order()
    path.to_hilbert(q.to(DEV), k.to(DEV), v.to(DEV))
    path.route(w.p, w.k)
    cnt = path.kv_count.clone()
    cnt[1, group:2 * group] = 0                     # head 1, tile 1: nothing kept
    tph = (path.nb + group - 1) // group
    T = w.heads * tph
    tiles = list(range(T))
    if layout == "one_list":
        W, lists = 4, [tiles, [], [], []]
    elif layout == "round_robin":
        W, lists = 3, [tiles[i::3] for i in range(3)]
    elif layout == "reversed":
        W, lists = 2, [tiles[::-1][:2], tiles[::-1][2:]]
    else:
        W, lists = T + 5, [[t] for t in tiles] + [[] for _ in range(5)]
    off = np.zeros(W + 1, dtype=np.int32)
    off[1:] = np.cumsum([len(x) for x in lists])
    wt = np.array([t for x in lists for t in x], dtype=np.int32)
    off_t = torch.from_numpy(off).to(DEV)
    wt_t = torch.from_numpy(wt).to(DEV)
    outs = []
    claims = torch.full((W,), -7, dtype=torch.int32, device=DEV)
    for use in (False, True):
        path.oh.fill_(float("nan"))
        _lib.sparse_attn(path.qh, path.kh, path.vh, path.oh, w.block, cnt, path.kv_index,
                         off_t, wt_t, W, v_tiles=True, group=group,
                         claims=claims if use else None)
        torch.cuda.synchronize()
        outs.append(path.oh.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    got = to_np(outs[1])
    assert (got[1, group * w.block:2 * group * w.block] == 0).all()
    c = claims.cpu().numpy()
    assert (c >= np.diff(off)).all()                 # every list was drained
    perm = path.perm.cpu().numpy()
    qh, kh, vh = (ort.permute_rows(to_np(x).astype(np.float64), perm) for x in (q, k, v))
    cn = cnt.cpu().numpy()
    kept_tiles = [(h, i) for h in range(w.heads) for i in range(path.nb) if cn[h, i] > 0]
    ref = oat.block_sparse_attention(qh, kh, vh, w.block, cn, path.kv_index.cpu().numpy(),
                                     tiles=kept_tiles)
    keep = ~np.isnan(ref)
    err = attn_errors(got[keep], ref[keep])
    assert err["max_abs"] <= TOL["bf16"]["max_abs"] and err["rel_l2"] <= TOL["bf16"]["rel_l2"], err


def test_rerun_is_bitwise_deterministic():
    w = workload("mid_bf16")
    say("determinism mid_bf16")
    q, k, v, _ = synth.make_inputs(w, "cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, device=DEV)
    outs = []
    for _ in range(2):
        o = path.run(q, k, v, w.p, w.k)
        torch.cuda.synchronize()
        outs.append([x.clone() for x in (o, path.mask, path.kv_index, path.worker_tiles,
                                         path.worker_offsets)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    # balanced and head-major launches run the same per-tile arithmetic
    path.attend(balanced=False)
    torch.cuda.synchronize()
    o2 = torch.empty_like(q)
    path.to_tokens(o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, outs[0][0])


def test_timing_records_every_worker():
    w = workload("mid_bf16")
    say("timing mid_bf16")
    q, k, v, _ = synth.make_inputs(w, "cpu")
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, n_workers=5, device=DEV)
    path.run(q.to(DEV), k.to(DEV), v.to(DEV), w.p, w.k)
    torch.cuda.synchronize()
    t = path.timing.cpu().numpy().astype(np.uint64)
    assert (t[:, 1] >= t[:, 0]).all() and (t[:, 0] > 0).all()
    # every worker ran inside one kernel launch: the spans overlap
    assert t[:, 0].max() <= t[:, 1].min() + 10_000_000


def test_attn_workers_is_a_multiple_of_the_cus():
    say("attn_workers")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for v_tiles in (True, False):
        for group in (1, 2, 3) if v_tiles else (1, 2):
            w = _lib.attn_workers(torch.bfloat16, 128, 128, v_tiles, group)
            assert w >= cus and w % cus == 0
    assert _lib.attn_workers(torch.float32, 64, 16, False) % cus == 0
