"""GPU regression test: run-time claims over runs of single-union-block tiles.

With claims on, the persistent kernels for tiles of two or three q-blocks post
claimed list positions in an LDS ring (its ordering is modelled on the CPU in test_claim_ring_model.py).
Runs of consecutive tiles with a single union block are the case that needs
that ordering: a Top-k floor of 0 or 1 makes them (the floor is optional
protection, aixai.ru FVAttn post, "Sparse-routing frontend"), and so does a
sequence no longer than one block (nB = 1).  Each case runs with tiles of two
and of three q-blocks, with one and two workers, with claims and with the
static lists; the outputs must be equal bit for bit, and within the attention
tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_11_amd import _lib
from oracle import attention as oat
from tests.parity import TOL, attn_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BLOCK = 128
D = 128


def say(msg):
    print(msg, flush=True)


def _lists(T, W, layout):
    tiles = list(range(T))
    if W == 1:
        return [tiles]
    if layout == "one_sided":                  # worker 1 takes everything by claims
        return [tiles, []]
    return [tiles[0::2], tiles[1::2]]


def _case(name, G):
    """(H, n, kv_count, kv_index) of a hand-made case; tiles hold q-blocks
    G*m .. G*m + G - 1 of a head."""
    if name == "nb1":
        H, n = 40, 100                          # one short block per head
        nb = 1
        cnt = np.ones((H, nb), dtype=np.int32)
        idx = np.zeros((H, nb, nb), dtype=np.int32)
        return H, n, cnt, idx
    H, n = 6, 8 * BLOCK - 37                    # ragged last block (91 keys)
    nb = 8
    cnt = np.ones((H, nb), dtype=np.int32)
    idx = np.zeros((H, nb, nb), dtype=np.int32)
    for h in range(H):
        for m in range((nb + G - 1) // G):
            j = (3 * h + 5 * m) % nb             # the tile's q-blocks keep the same block
            for i in range(G * m, min(nb, G * m + G)):
                idx[h, i, 0] = j
    if name == "mixed":
        # single-block runs broken by a pair with nothing kept, a pair whose
        # halves keep one block each (two union blocks) and a longer pair
        cnt[1, 2:4] = 0
        idx[2, 4, 0], idx[2, 5, 0] = 1, 6
        cnt[4, 0], cnt[4, 1] = 3, 2
        idx[4, 0, :3] = [0, 2, 7]
        idx[4, 1, :2] = [2, 5]
    return H, n, cnt, idx


@pytest.mark.parametrize("name", ["single", "mixed", "nb1"])
@pytest.mark.parametrize("W,layout", [(1, "one"), (2, "split"), (2, "one_sided")])
@pytest.mark.parametrize("G", [2, 3])
def test_claims_over_single_block_tiles(name, W, layout, G):
    say(f"claim ring {name} W={W} {layout} group={G}")
    H, n, cnt, idx = _case(name, G)
    nb = cnt.shape[1]
    tph = (nb + G - 1) // G
    g = torch.Generator().manual_seed(11)
    q = (torch.randn((H, n, D), generator=g) * 2).to(torch.bfloat16)
    k = (torch.randn((H, n, D), generator=g) * 2).to(torch.bfloat16)
    v = torch.randn((H, n, D), generator=g).to(torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    vt = torch.empty((H, nb, D, BLOCK), dtype=torch.bfloat16, device=DEV)
    _lib.pack_v(vd, vt, torch.arange(n, dtype=torch.int32, device=DEV), BLOCK)
    lists = _lists(H * tph, W, layout)
    off = np.zeros(W + 1, dtype=np.int32)
    off[1:] = np.cumsum([len(x) for x in lists])
    wt = np.array([t for x in lists for t in x], dtype=np.int32)
    off_t, wt_t = torch.from_numpy(off).to(DEV), torch.from_numpy(wt).to(DEV)
    cnt_t, idx_t = torch.from_numpy(cnt).to(DEV), torch.from_numpy(idx).to(DEV)
    claims = torch.full((W,), -7, dtype=torch.int32, device=DEV)
    outs = []
    for use in (False, True):
        o = torch.full((H, n, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        _lib.sparse_attn(qd, kd, vt, o, BLOCK, cnt_t, idx_t, off_t, wt_t, W,
                         v_tiles=True, group=G, claims=claims if use else None)
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert (claims.cpu().numpy() >= np.diff(off)).all()       # every list drained
    got = outs[1].float().cpu().numpy()
    kept = [(h, i) for h in range(H) for i in range(nb) if cnt[h, i] > 0]
    empty = [(h, i) for h in range(H) for i in range(nb) if cnt[h, i] == 0]
    for h, i in empty:
        assert (got[h, i * BLOCK:min(n, (i + 1) * BLOCK)] == 0).all()
    ref = oat.block_sparse_attention(q.float().numpy().astype(np.float64),
                                     k.float().numpy().astype(np.float64),
                                     v.float().numpy().astype(np.float64),
                                     BLOCK, cnt, idx, tiles=kept)
    keep = ~np.isnan(ref)
    assert not np.isnan(got[keep]).any()
    err = attn_errors(got[keep], ref[keep])
    tol = TOL["bf16"]
    assert err["max_abs"] <= tol["max_abs"] and err["rel_l2"] <= tol["rel_l2"], err
