"""Oracle steps 2-5: reorder, block pooling, pooled scores, Top-p + Top-k cut.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * routing estimates how important each key block is for a query block from
    pooled Q and K, and that one routing pass yields the mask and each head's
    density (PaperDaily FVAttn article, method section; aixai.ru FVAttn post,
    section "Sparse-routing frontend");
  * Top-p keeps, per query block, key blocks in order of importance until
    their accumulated importance reaches the threshold p, so a concentrated
    head keeps few blocks and a flat head keeps many (aixai.ru post, section
    "Top-p vs Top-k"; PaperDaily article, introduction of Top-p routing);
  * the Top-k safety floor always keeps at least the k most important blocks
    (PaperDaily article, method section; arXiv abstract);
  * a head's load is its number of kept sparse blocks, the unit of work
    (aixai.ru post, section "Runtime Load Balancing (RLB)").

Readings taken where the pages are silent (listed in the design notes):
  * pooling is the arithmetic mean over the block's true rows (the last block
    may be short);
  * importance of key block j for query block i is softmax_j of
    (qbar_i . kbar_j) / sqrt(d), so each row sums to one and p is a fraction
    of that mass;
  * blocks are ranked by (importance descending, index ascending); n_p is the
    smallest prefix whose accumulated mass is >= p (all blocks if p >= 1 or if
    no prefix reaches p); n_keep = min(nB, max(n_p, k));
  * head density = kept blocks / nB**2.

All arithmetic here is float64.  Pins (tests/test_oracle_route.py): pooling of
rows with a known mean, a hand-computed 2x2 score table, softmax invariants,
the closed forms for uniform rows (nB = 8) and a dominant block, brute force
over all subsets for nB <= 10, and the row invariants (floor, mass, minimality,
top-set).  The importance formula itself is a reading: parity of the mask
against the method as published is unpinned (no page prints a mask).
"""
from __future__ import annotations

import math

import numpy as np


def num_blocks(n: int, block: int) -> int:
    return (n + block - 1) // block


def block_sizes(n: int, block: int) -> np.ndarray:
    """True row count n_j of each block j (the last block may be short)."""
    nb = num_blocks(n, block)
    sizes = np.full(nb, block, dtype=np.int64)
    sizes[-1] = n - (nb - 1) * block
    return sizes


def permute_rows(x: np.ndarray, index: np.ndarray) -> np.ndarray:
    """dst[h, r, :] = src[h, index[r], :]."""
    return np.asarray(x)[:, np.asarray(index, dtype=np.int64), :]


def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of each block's rows: [H, n, d] -> [H, nB, d], float64."""
    H, n, d = x.shape
    nb = num_blocks(n, block)
    out = np.empty((H, nb, d), dtype=np.float64)
    for j in range(nb):
        rows = x[:, j * block:min(n, (j + 1) * block), :].astype(np.float64)
        out[:, j, :] = rows.sum(axis=1) / rows.shape[1]
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """z[h, i, j] = qbar[h, i] . kbar[h, j] / sqrt(d)."""
    d = qbar.shape[-1]
    return np.einsum("hid,hjd->hij", qbar.astype(np.float64),
                     kbar.astype(np.float64)) / math.sqrt(d)


def row_softmax(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, shifted by the row maximum."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def rank_blocks(P_row: np.ndarray) -> np.ndarray:
    """Key-block indices ordered by (importance descending, index ascending)."""
    j = np.arange(P_row.shape[0])
    return np.lexsort((j, -np.asarray(P_row, dtype=np.float64)))


def top_p_count(P_sorted: np.ndarray, p: float) -> int:
    """Smallest prefix length m with accumulated mass >= p (all if none)."""
    nb = P_sorted.shape[0]
    if p >= 1.0:
        return nb
    acc = 0.0
    for m in range(nb):
        acc += float(P_sorted[m])
        if acc >= p:
            return m + 1
    return nb


def select_row(P_row: np.ndarray, p: float, k: int):
    """Kept key blocks of one query-block row.

    Returns (kept ascending int64 array, n_p, order) where order is the
    importance ranking used for the cut.
    """
    nb = P_row.shape[0]
    order = rank_blocks(P_row)
    n_p = top_p_count(P_row[order], p)
    n_keep = min(nb, max(n_p, k))
    kept = np.sort(order[:n_keep])
    return kept, n_p, order


def route_from_probs(P: np.ndarray, p: float, k: int):
    """Mask and kept-block lists from the importance table P [H, nB, nB]."""
    H, nb, _ = P.shape
    mask = np.zeros((H, nb, nb), dtype=np.uint8)
    kv_count = np.zeros((H, nb), dtype=np.int32)
    kv_index = np.full((H, nb, nb), -1, dtype=np.int32)
    for h in range(H):
        for i in range(nb):
            kept, _, _ = select_row(P[h, i], p, k)
            mask[h, i, kept] = 1
            kv_count[h, i] = kept.shape[0]
            kv_index[h, i, :kept.shape[0]] = kept
    head_load = kv_count.astype(np.int64).sum(axis=1)
    head_density = head_load.astype(np.float64) / float(nb * nb)
    return mask, kv_count, kv_index, head_load, head_density


def route(qh: np.ndarray, kh: np.ndarray, block: int, p: float, k: int):
    """Full routing on Hilbert-ordered Q, K [H, n, d].

    Returns a dict with qbar, kbar, z, P, mask, kv_count, kv_index, head_load,
    head_density.
    """
    if not (p > 0.0):
        raise ValueError("p must be > 0")
    if k < 0:
        raise ValueError("k must be >= 0")
    qbar = pool_blocks(qh, block)
    kbar = pool_blocks(kh, block)
    z = block_scores(qbar, kbar)
    P = row_softmax(z)
    mask, kv_count, kv_index, head_load, head_density = route_from_probs(P, p, k)
    return dict(qbar=qbar, kbar=kbar, z=z, P=P, mask=mask, kv_count=kv_count,
                kv_index=kv_index, head_load=head_load,
                head_density=head_density)
