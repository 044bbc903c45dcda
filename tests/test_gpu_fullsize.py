"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default persistent worker count, V key-block tiles, q-block
pairs, two-level LPT lists over the XCDs, run-time claims).

At these sizes the oracle still runs every integer step in full (Hilbert
order, routing of every row of every head, the LPT schedule), while the
attention is compared on sampled tiles, which the oracle computes one by one:
the last (ragged) q-block, the heaviest and the lightest tiles, tiles of the
flat heads, and seeded random ones.
"""

import numpy as np
import pytest
import torch

from block_sparse_attention_11_amd import synth
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


def head_f64(x, h):
    return x[h].float().cpu().numpy().astype(np.float64)


def run_full(w, p=None, seed=None, r_override=None, group=None):
    p = w.p if p is None else p
    if seed is not None:
        w = w.with_(seed=seed)
    q, k, v, _ = synth.make_inputs(w, DEV, r_override=r_override)
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, device=DEV, group=group)
    out = path.run(q, k, v, p, w.k)
    torch.cuda.synchronize()
    return path, q, k, v, out, p


def sample_tiles(path, n_random=6, seed=7):
    kvc = path.kv_count.cpu().numpy()
    H, nb = kvc.shape
    flat = np.unravel_index(np.arange(H * nb), (H, nb))
    costs = kvc.reshape(-1)
    picks = {(0, nb - 1), (H - 1, nb - 1), (H - 1, 0)}
    picks.add(tuple(int(x) for x in np.unravel_index(int(costs.argmax()), (H, nb))))
    picks.add(tuple(int(x) for x in np.unravel_index(int(costs.argmin()), (H, nb))))
    rng = np.random.default_rng(seed)
    for t in rng.choice(H * nb, size=n_random, replace=False):
        picks.add((int(flat[0][t]), int(flat[1][t])))
    return sorted(picks)


def oracle_rows(x, h, perm):
    """Head h of x (token order) in the oracle's Hilbert order, float64 [1, n, d]."""
    return ort.permute_rows(head_f64(x, h)[None], perm)


def check_gather(path, q, k, heads):
    """The GPU's Hilbert-ordered Q and K of the given heads equal, byte for
    byte, the oracle's permutation of the original rows."""
    perm, _ = ohb.hilbert_order(*path.grid)
    bits = torch.int16 if q.dtype == torch.bfloat16 else torch.int32
    for h in heads:
        for src, got in ((q, path.qh), (k, path.kh)):
            want = ort.permute_rows(src[h:h + 1].cpu().view(bits).numpy(), perm)
            assert np.array_equal(got[h:h + 1].cpu().view(bits).numpy(), want), h
    say(f"  Q/K gather bytes equal the oracle's on heads {list(heads)}")


def check_route(path, w, p, heads, q, k):
    """Every row of the given heads against the oracle's routing of the
    original Q/K in the oracle's Hilbert order; invariants on every head."""
    nb = path.nb
    perm, _ = ohb.hilbert_order(*w.grid)
    gc = path.kv_count.cpu().numpy()
    gi = path.kv_index.cpu().numpy()
    total = {"rows": 0, "exact": 0, "count": 0, "order": 0, "unexplained": 0}
    for h in heads:
        ora = ort.route(oracle_rows(q, h, perm), oracle_rows(k, h, perm), w.block, p, w.k)
        stats, bad = classify_rows(ora["P"], p, w.k, gc[h:h + 1], gi[h:h + 1],
                                   ora["kv_count"], ora["kv_index"])
        for key in total:
            total[key] += stats[key]
        assert stats["unexplained"] == 0, (h, bad[:5])
    say(f"  mask rows over heads {list(heads)}: {total}")
    assert (gc >= min(w.k, nb)).all() and (gc <= nb).all()
    load = path.head_load.cpu().numpy()
    assert np.array_equal(load, gc.astype(np.int64).sum(1))
    dens = path.head_density.cpu().numpy()
    assert np.array_equal(dens, (load / float(nb * nb)).astype(np.float32))
    # the mask bits and the kept lists describe the same sets
    mask = path.mask.cpu().numpy()
    assert np.array_equal(mask.sum(-1, dtype=np.int64), gc)
    for h in range(0, w.heads, max(1, w.heads // 4)):
        for i in range(0, nb, max(1, nb // 16)):
            assert np.flatnonzero(mask[h, i]).tolist() == gi[h, i, :gc[h, i]].tolist()


def check_schedule(path):
    costs = olpt.group_costs(path.kv_count.cpu().numpy(), path.group)
    if path.worker_groups > 1:
        ref = olpt.lpt_schedule_grouped(costs.reshape(path.heads, -1), path.n_workers,
                                        path.worker_groups, tile_order=path.tile_order)
    else:
        ref = olpt.lpt_schedule(costs, path.n_workers, tile_order=path.tile_order)
    got = (path.lpt_order, path.worker_offsets, path.worker_tiles, path.worker_load)
    for g, r, what in zip(got, ref, ("order", "offsets", "tiles", "loads")):
        assert np.array_equal(g.cpu().numpy(), r), what


def check_attention(path, w, q, k, v, out, tiles):
    """Sampled tiles against the oracle on the original Q/K/V in the oracle's
    Hilbert order, with the GPU's kept lists."""
    perm, _ = ohb.hilbert_order(*w.grid)
    gc = path.kv_count.cpu().numpy()
    gi = path.kv_index.cpu().numpy()
    worst = {"max_abs": 0.0, "rel_l2": 0.0}
    for h in sorted({t[0] for t in tiles}):
        qh, kh, vh = (oracle_rows(x, h, perm) for x in (q, k, v))
        outh = out[h].float().cpu().numpy()
        ohh = outh[perm]                    # Hilbert order
        for (hh, i) in tiles:
            if hh != h:
                continue
            r0, r1 = i * w.block, min(path.n, (i + 1) * w.block)
            ref = oat.block_sparse_attention_tile(qh, kh, vh, 0, i, w.block,
                                                  gi[h, i, :gc[h, i]])
            err = attn_errors(ohh[r0:r1], ref)
            for key in worst:
                worst[key] = max(worst[key], err[key])
            tol = TOL[w.dtype]
            assert err["max_abs"] <= tol["max_abs"] and err["rel_l2"] <= tol["rel_l2"], \
                (h, i, int(gc[h, i]), err)
    say(f"  attention on {len(tiles)} sampled tiles: worst {worst}")


@pytest.mark.parametrize("name,group", [("480p", None), ("720p", None), ("720p_sparse", None),
                                        ("720p", 2), ("720p", 3), ("720p_sparse", 3),
                                        ("480p", 3), ("720p_rank", None),
                                        ("long720p_sparse", None)])
def test_fullsize_path(name, group):
    w = synth.WORKLOADS[name]
    say(f"full-size path {name}: {w.heads} heads, grid {w.grid}, block {w.block}, "
        f"group {group}")
    path, q, k, v, out, p = run_full(w, group=group)
    say(f"  workers {path.n_workers}, group {path.group}, v_tiles {path.v_tiles}")
    perm, inv = ohb.hilbert_order(*w.grid)
    assert np.array_equal(path.perm.cpu().numpy(), perm)
    assert np.array_equal(path.inv_perm.cpu().numpy(), inv)
    H = w.heads
    heads = sorted({0, 1, H // 2, H - 1} | ({32, 39} if H == 40 else set()))
    check_gather(path, q, k, heads)
    check_route(path, w, p, heads, q, k)
    check_schedule(path)
    check_attention(path, w, q, k, v, out, sample_tiles(path))


def test_fullsize_480p_dense_control():
    """p = 1 keeps every block: the same kernels compute dense attention."""
    w = synth.WORKLOADS["480p"]
    say("full-size dense control 480p (p = 1)")
    path, q, k, v, out, p = run_full(w, p=1.0)
    gc = path.kv_count.cpu().numpy()
    assert (gc == path.nb).all()
    assert (path.head_density.cpu().numpy() == 1.0).all()
    check_schedule(path)
    check_attention(path, w, q, k, v, out, sample_tiles(path, n_random=4))


@pytest.mark.parametrize("name", ["long720p", "long720p_p90"])
def test_fullsize_long720p_steps(name):
    """Four steps of the long workload, s/K/E/V redrawn per step: routing,
    schedule and attention on fresh masks each step (all from one path
    object, as a sampler would run it), at Top-p 0.95 and 0.90."""
    w = synth.WORKLOADS[name]
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, device=DEV)
    perm, _ = ohb.hilbert_order(*w.grid)
    prev = None
    for step, r0 in synth.long_steps(w):
        say(f"{name} step {step} (p = {w.p})")
        ws = w.with_(seed=step)
        q, k, v, _ = synth.make_inputs(ws, DEV, r_override=r0)
        out = path.run(q, k, v, w.p, w.k)
        torch.cuda.synchronize()
        if step == 0:
            assert np.array_equal(path.perm.cpu().numpy(), perm)
        heads = [step, 39 - step]
        check_gather(path, q, k, heads)
        check_route(path, w, w.p, heads, q, k)
        check_schedule(path)
        check_attention(path, w, q, k, v, out, sample_tiles(path, n_random=3, seed=step))
        dens = path.head_density.cpu().numpy()
        if prev is not None:
            say(f"  density change vs previous step: max {np.abs(dens - prev).max():.4f}")
        prev = dens
        del q, k, v, out
