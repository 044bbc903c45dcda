"""Attention on tiled-V tensors larger than 2 GiB.

The tiled-V kernels address K and V one head at a time (a buffer descriptor
per head, 32-bit byte offsets inside it), so a tensor may exceed 2^31 bytes;
only one head of V tiles must fit in 4 GiB (`test_abi.py` checks the refusal
past it).  Here: 17 heads x 4095 key blocks of 128 x 128 in bf16,
2,281,138,560 bytes per tensor, one head past the 2^31 - 1 bytes that a
single 32-bit offset over the whole tensor could reach, with a ragged last
block.  Each q-block keeps itself and a mirrored block (one block where the
two coincide), so the last head's tail block, the highest offsets of every
tensor, is read.  Grid launch and the persistent launch with LPT lists and
run-time claims; sampled tiles against the plain float64 definition of
attention on the kept rows.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_11_amd import _lib
from oracle import attention as oat
from tests.parity import TOL, attn_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
H, NB, BLOCK, D = 17, 4095, 128, 128
N = NB * BLOCK - 37


def say(msg):
    print(msg, flush=True)


def kept_lists():
    i = torch.arange(NB, device=DEV)
    h = torch.arange(H, device=DEV)[:, None]
    a = i[None, :].expand(H, NB)
    b = (NB - 1 - i[None, :] + 3 * h) % NB
    lo, hi = torch.minimum(a, b), torch.maximum(a, b)
    cnt = torch.where(lo == hi, 1, 2).to(torch.int32)
    idx = torch.zeros((H, NB, NB), dtype=torch.int32, device=DEV)
    idx[:, :, 0] = lo.to(torch.int32)
    idx[:, :, 1] = torch.where(lo == hi, 0, hi).to(torch.int32)
    return cnt.contiguous(), idx


def rows(x, h, blocks):
    r = np.concatenate([np.arange(j * BLOCK, min(N, (j + 1) * BLOCK)) for j in blocks])
    t = torch.from_numpy(r).to(DEV)
    return x[h].index_select(0, t).float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("mode", ["grid", "persistent"])
def test_attention_on_tiled_tensors_past_2gib(mode):
    assert (H - 1) * NB * BLOCK * D * 2 <= 0x7FFFFFFF < H * NB * BLOCK * D * 2
    say(f"tiled tensors past 2 GiB: {H} heads, n={N}, {mode}")
    g = torch.Generator(device=DEV).manual_seed(11)
    q = torch.randn((H, N, D), generator=g, device=DEV, dtype=torch.bfloat16)
    k = torch.randn((H, N, D), generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((H, N, D), generator=g, device=DEV, dtype=torch.bfloat16)
    vt = torch.empty((H, NB, D, BLOCK), dtype=torch.bfloat16, device=DEV)
    _lib.pack_v(v, vt, torch.arange(N, dtype=torch.int32, device=DEV), BLOCK)
    cnt, idx = kept_lists()
    o = torch.full((H, N, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    kw = {}
    if mode == "persistent":
        W = _lib.attn_workers(torch.bfloat16, D, BLOCK, True, 2)
        tiles = H * ((NB + 1) // 2)
        i32 = dict(dtype=torch.int32, device=DEV)
        off, wt = torch.empty(W + 1, **i32), torch.empty(tiles, **i32)
        ws = torch.empty(_lib.schedule_workspace_size(H, NB, W), dtype=torch.uint8, device=DEV)
        _lib.schedule(cnt, W, torch.empty(tiles, **i32), off, wt,
                      torch.empty(W, dtype=torch.int64, device=DEV), ws, group=2)
        kw = dict(worker_offsets=off, worker_tiles=wt, n_workers=W,
                  claims=torch.zeros(W, **i32))
    _lib.sparse_attn(q, k, vt, o, BLOCK, cnt, idx, v_tiles=True, group=2, **kw)
    torch.cuda.synchronize()
    del vt
    assert not torch.isnan(o).any()
    c, x = cnt.cpu().numpy(), idx[:, :, :2].cpu().numpy()
    gen = np.random.default_rng(5)
    sample = [(0, 0), (0, NB - 1), (H - 1, 0), (H - 1, NB - 1), (H - 1, NB - 2),
              (H - 1, (NB - 1) // 2), (7, 1000)]
    sample += [(int(gen.integers(H)), int(gen.integers(NB))) for _ in range(5)]
    tol = TOL["bf16"]
    for h, i in sample:
        kept = x[h, i, :c[h, i]].tolist()
        ref = oat.dense_attention(rows(q, h, [i])[None], rows(k, h, kept)[None],
                                  rows(v, h, kept)[None])[0]
        got = rows(o, h, [i])
        err = attn_errors(got, ref)
        assert err["max_abs"] <= tol["max_abs"] and err["rel_l2"] <= tol["rel_l2"], (h, i, kept, err)
    say(f"  {len(sample)} tiles within {tol}")
