"""Pins for the oracle's block-sparse attention (CPU only).

With every block kept, sparse attention is ordinary dense attention (the
FlashAttention baseline of the aixai.ru FVAttn post, "Attention: 4.41x
over FlashAttention"); with a mask it skips exactly the dropped blocks.  The
oracle is checked against torch's own scaled_dot_product_attention routine
on the CPU in float64, a separate implementation.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as at
from oracle import hilbert as hb
from oracle import route as rt


def sdpa(q, k, v, mask=None):
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None]
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))[None]
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    return out[0].numpy()


@pytest.mark.parametrize("grid,block,d,H", [((2, 8, 8), 16, 64, 1),
                                            ((3, 5, 7), 16, 32, 2),
                                            ((4, 6, 5), 32, 16, 2)])
def test_dense_through_hilbert_equals_sdpa(grid, block, d, H):
    rng = np.random.default_rng(7)
    n = grid[0] * grid[1] * grid[2]
    q, k, v = (rng.normal(size=(H, n, d)) for _ in range(3))
    perm, inv = hb.hilbert_order(*grid)
    qh, kh, vh = (rt.permute_rows(x, perm) for x in (q, k, v))
    nb = rt.num_blocks(n, block)
    cnt = np.full((H, nb), nb, dtype=np.int32)
    idx = np.tile(np.arange(nb, dtype=np.int32), (H, nb, 1))
    oh = at.block_sparse_attention(qh, kh, vh, block, cnt, idx)
    o = at.unpermute_rows(oh, perm)
    assert np.allclose(o, sdpa(q, k, v), rtol=1e-12, atol=1e-12)
    assert np.allclose(o, rt.permute_rows(oh, inv), rtol=0, atol=0)
    assert np.allclose(at.dense_attention(q, k, v), sdpa(q, k, v), atol=1e-12)


def test_masked_equals_sdpa_with_token_mask():
    rng = np.random.default_rng(8)
    H, n, d, B = 2, 105, 16, 16
    nb = rt.num_blocks(n, B)
    q, k, v = (rng.normal(size=(H, n, d)) for _ in range(3))
    out = rt.route(q, k, B, 0.6, 2)
    o = at.block_sparse_attention(q, k, v, B, out["kv_count"], out["kv_index"])
    blk = np.arange(n) // B
    for h in range(H):
        tok_mask = out["mask"][h][blk][:, blk].astype(bool)
        ref = sdpa(q[h:h + 1], k[h:h + 1], v[h:h + 1], tok_mask[None])[0]
        assert np.allclose(o[h], ref, atol=1e-12)
    assert nb == 7


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(9)
    H, n, d, B = 1, 70, 8, 16
    q, k = rng.normal(size=(2, H, n, d)) * 3
    v = np.broadcast_to(np.arange(d, dtype=np.float64), (H, n, d)).copy()
    out = rt.route(q, k, B, 0.3, 1)
    o = at.block_sparse_attention(q, k, v, B, out["kv_count"], out["kv_index"])
    assert np.allclose(o, v, atol=1e-12)


def test_single_kept_block_is_softmax_over_it():
    rng = np.random.default_rng(10)
    H, n, d, B = 1, 64, 8, 16
    q, k, v = rng.normal(size=(3, H, n, d))
    cnt = np.ones((1, 4), dtype=np.int32)
    idx = np.zeros((1, 4, 4), dtype=np.int32)
    idx[0, :, 0] = [2, 0, 3, 1]
    o = at.block_sparse_attention(q, k, v, B, cnt, idx)
    for i, j in enumerate([2, 0, 3, 1]):
        s = q[0, i * B:(i + 1) * B] @ k[0, j * B:(j + 1) * B].T / math.sqrt(d)
        pr = np.exp(s - s.max(1, keepdims=True))
        pr /= pr.sum(1, keepdims=True)
        assert np.allclose(o[0, i * B:(i + 1) * B], pr @ v[0, j * B:(j + 1) * B])


def test_kept_flops():
    H, n, d, B = 2, 105, 8, 16
    nb = 7
    cnt = np.full((H, nb), nb, dtype=np.int32)
    idx = np.tile(np.arange(nb, dtype=np.int32), (H, nb, 1))
    assert at.kept_flops(cnt, idx, n, B, d) == 4 * H * n * n * d
    cnt1 = np.ones((H, nb), dtype=np.int32)
    idx1 = np.zeros((H, nb, nb), dtype=np.int32)
    idx1[:, :, 0] = nb - 1          # the 9-row tail block
    assert at.kept_flops(cnt1, idx1, n, B, d) == 4 * H * n * 9 * d
