"""Routing from pooled means (fvattn_route_pooled) at every size class of the
per-row sort, through the C ABI, against the oracle.

The sort keeps nB keys per row spread over 256 threads, 1, 2, 4, 8 or 16 per
thread, so its code differs by size class.  Each class is run at its lower
edge, its upper edge and one past it, up to the largest supported nB = 4096.
The pooled means are given (seeded, with per-row scales from near-uniform to
sharply peaked importance rows); the oracle forms the scores and importances
from the same fp32 means in float64 and selects each sampled row.  Rows are
compared with the near-tie protocol of the other routing tests; the mask, the
kept lists, the loads and the densities are checked for consistency on every
row.  p = 1 must keep every block of every row.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_11_amd import _lib
from oracle import route as ort
from tests.parity import classify_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BLOCK = 16
D = 32
NBS = [1, 2, 3, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049,
       4095, 4096]


def say(msg):
    print(msg, flush=True)


def pooled_inputs(nb, heads, seed, d=D):
    g = np.random.default_rng(seed)
    qbar = g.standard_normal((heads, nb, d)).astype(np.float32)
    kbar = g.standard_normal((heads, nb, d)).astype(np.float32)
    # row scales 0.05 .. 8: from nearly uniform importances to a few dominant blocks
    scale = np.exp(g.uniform(math.log(0.05), math.log(8.0), (heads, nb, 1)))
    return (qbar * scale).astype(np.float32), kbar


def run(qbar, kbar, n, p, k):
    H, nb, d = qbar.shape
    i32 = dict(dtype=torch.int32, device=DEV)
    out = dict(mask=torch.empty((H, nb, nb), dtype=torch.uint8, device=DEV),
               kv_count=torch.empty((H, nb), **i32),
               kv_index=torch.empty((H, nb, nb), **i32),
               head_load=torch.empty(H, dtype=torch.int64, device=DEV),
               head_density=torch.empty(H, dtype=torch.float32, device=DEV))
    ws = torch.empty(_lib.route_workspace_size(H, n, d, BLOCK), dtype=torch.uint8, device=DEV)
    _lib.route_pooled(torch.from_numpy(qbar).to(DEV), torch.from_numpy(kbar).to(DEV), n,
                      BLOCK, p, k, out["mask"], out["kv_count"], out["kv_index"],
                      out["head_load"], out["head_density"], ws)
    torch.cuda.synchronize()
    return {key: t.cpu().numpy() for key, t in out.items()}


def check_consistent(r, nb, k):
    gc, gi, mask = r["kv_count"], r["kv_index"], r["mask"]
    H = gc.shape[0]
    assert (gc >= min(k, nb)).all() and (gc <= nb).all()
    assert np.array_equal(mask.sum(-1, dtype=np.int64), gc.astype(np.int64))
    # every kept list strictly ascending inside [0, nB) and equal to its mask row
    cols = np.arange(nb)
    valid = cols[None, None, :] < gc[..., None]
    lists = np.where(valid, gi, -1)
    assert (np.where(valid, gi, 0) >= 0).all() and (np.where(valid, gi, 0) < nb).all()
    inc = np.diff(np.where(valid, gi, np.iinfo(np.int32).max), axis=-1)
    assert (inc[valid[..., 1:]] > 0).all()
    rebuilt = np.zeros_like(mask)
    hh, ii, cc = np.nonzero(valid)
    rebuilt[hh, ii, lists[hh, ii, cc]] = 1
    assert np.array_equal(rebuilt, mask)
    load = gc.astype(np.int64).sum(1)
    assert np.array_equal(r["head_load"], load)
    assert np.array_equal(r["head_density"], (load / float(nb * nb)).astype(np.float32))
    return H


CASES = [(nb, D) for nb in NBS] + [(3, 4), (591, 4), (3, 256), (591, 256), (2049, 256)]


@pytest.mark.parametrize("nb,d", CASES)
def test_select_size_classes(nb, d):
    """d from the smallest (4) to the largest (256) pooled width the ABI takes."""
    heads = 2 if nb <= 1024 else 1
    n = nb * BLOCK - (5 if nb > 1 else 3)          # ragged last block
    p, k = 0.9, 4
    say(f"select nB={nb} d={d} heads={heads} n={n} p={p} k={k}")
    qbar, kbar = pooled_inputs(nb, heads, seed=nb + d, d=d)
    r = run(qbar, kbar, n, p, k)
    check_consistent(r, nb, k)
    g = np.random.default_rng(1000 + nb)
    rows = np.arange(nb) if nb <= 600 else np.unique(np.concatenate(
        [np.arange(8), np.arange(nb - 8, nb), g.choice(nb, 80, replace=False)]))
    for h in range(heads):
        P = ort.row_softmax(ort.block_scores(qbar[h:h + 1, rows], kbar[h:h + 1]))
        oc = np.zeros((1, rows.size), dtype=np.int32)
        oi = np.full((1, rows.size, nb), -1, dtype=np.int32)
        for x in range(rows.size):
            kept, _, _ = ort.select_row(P[0, x], p, k)
            oc[0, x] = kept.size
            oi[0, x, :kept.size] = kept
        stats, bad = classify_rows(P, p, k, r["kv_count"][h:h + 1, rows],
                                   r["kv_index"][h:h + 1, rows], oc, oi)
        say(f"  head {h}: {stats}")
        assert stats["unexplained"] == 0, [int(rows[i]) for _, i in bad[:5]]
    # the rows span sparse and dense decisions
    if nb >= 255:
        assert r["kv_count"].min() < nb // 4 and r["kv_count"].max() > nb // 2


@pytest.mark.parametrize("nb", [257, 2049, 4096])
def test_select_p_one_keeps_every_block(nb):
    n = nb * BLOCK
    say(f"select nB={nb} p=1")
    qbar, kbar = pooled_inputs(nb, 1, seed=7 * nb)
    r = run(qbar, kbar, n, 1.0, 0)
    check_consistent(r, nb, 0)
    assert (r["kv_count"] == nb).all()
    assert (r["kv_index"] == np.arange(nb, dtype=np.int32)[None, None, :]).all()
