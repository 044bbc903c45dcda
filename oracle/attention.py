"""Oracle step 7: softmax attention over the kept key blocks only.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: sparse attention computes only the (query block, key
block) interactions the mask keeps and skips the rest (aixai.ru FVAttn post,
"What is sparse attention in video transformers" and "Top-p vs Top-k"; the
arXiv abstract on the mlsanity.com index page).  With every block kept the
result is ordinary dense attention, the FlashAttention baseline the pages
compare against.

Readings taken: no causal mask (bidirectional video self-attention); scale
1/sqrt(d); batch folded into heads; a query row attends to every row of every
kept key block (the last block may be short); output dtype = input dtype.

This is the plain definition: for each query block i of head h the kept keys
are gathered, scores are formed, a float64 softmax is taken over them and the
values are averaged.  Pins (tests/test_oracle_attention.py): with all blocks
kept and the Hilbert permutation undone it equals torch's
scaled_dot_product_attention on the original token order; a masked case
equals that routine with the equivalent boolean mask; constant V rows give
that constant; a single kept key block reduces to ordinary softmax over it.
"""
from __future__ import annotations

import math

import numpy as np


def block_sparse_attention_tile(qh, kh, vh, h: int, i: int, block: int,
                                kept_blocks, scale: float | None = None):
    """Output rows of query block i of head h, float64 [n_i, d]."""
    n = qh.shape[1]
    d = qh.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r0, r1 = i * block, min(n, (i + 1) * block)
    q = qh[h, r0:r1].astype(np.float64)
    rows = np.concatenate([np.arange(j * block, min(n, (j + 1) * block))
                           for j in kept_blocks])
    k = kh[h, rows].astype(np.float64)
    v = vh[h, rows].astype(np.float64)
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ v


def block_sparse_attention(qh, kh, vh, block: int, kv_count, kv_index,
                           scale: float | None = None, tiles=None):
    """Block-sparse attention on Hilbert-ordered [H, n, d] tensors.

    kv_count [H, nB] and kv_index [H, nB, nB] (ascending, first kv_count
    valid).  tiles: optional iterable of (h, i) to compute; other rows are
    left as NaN.  Returns float64 [H, n, d].
    """
    H, n, d = qh.shape
    nb = (n + block - 1) // block
    out = np.full((H, n, d), np.nan, dtype=np.float64)
    if tiles is None:
        tiles = [(h, i) for h in range(H) for i in range(nb)]
    for h, i in tiles:
        kept = np.asarray(kv_index[h, i, :kv_count[h, i]])
        out[h, i * block:min(n, (i + 1) * block)] = block_sparse_attention_tile(
            qh, kh, vh, h, i, block, kept, scale)
    return out


def unpermute_rows(oh: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """O[h, perm[r]] = Oh[h, r]: back to the original token order."""
    out = np.empty_like(oh)
    out[:, np.asarray(perm, dtype=np.int64), :] = oh
    return out


def dense_attention(q, k, v, scale: float | None = None) -> np.ndarray:
    """softmax(q k^T * scale) v per head, float64, no blocking."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    out = np.empty_like(q)
    for h in range(q.shape[0]):
        s = (q[h] @ k[h].T) * scale
        s -= s.max(axis=1, keepdims=True)
        e = np.exp(s)
        out[h] = (e / e.sum(axis=1, keepdims=True)) @ v[h]
    return out


def kept_flops(kv_count, kv_index, n: int, block: int, d: int) -> int:
    """Sum over kept (h, i, j) of 4 * n_i * n_j * d with true block sizes."""
    nb = (n + block - 1) // block
    sizes = np.full(nb, block, dtype=np.int64)
    sizes[-1] = n - (nb - 1) * block
    total = 0
    H = kv_count.shape[0]
    for h in range(H):
        for i in range(nb):
            c = int(kv_count[h, i])
            total += 4 * int(sizes[i]) * int(sizes[kv_index[h, i, :c]].sum()) * d
    return total
