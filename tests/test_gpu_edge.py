"""The whole path (Hilbert order, fused gather + pooling, routing, schedule,
persistent attention with claims, O stored in token order) on degenerate
shapes, against the oracle: every routed row, the schedule bit for bit, and
attention on every tile.

Cases: a single token; a sequence shorter than one 128-key block (the
second 64-key half of the only block is all padding); 65 tokens (one valid
key in that half); a Top-p threshold so small that one block per row
passes, with no Top-k floor; p = 1 (dense); a Top-k floor above the block
count; fp32 inputs on the scalar kernel with a single token.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_11_amd import synth
from block_sparse_attention_11_amd.pipeline import FVAttnPath
from tests.test_gpu_fullsize import (check_attention, check_gather, check_route,
                                     check_schedule)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

W = synth.Workload
CASES = {
    "one_token": W("one_token", 2, 128, (1, 1, 1), 128, 0.95, 8, "bf16"),
    "short_seq": W("short_seq", 2, 128, (1, 5, 9), 128, 0.95, 8, "bf16"),
    "tail_65": W("tail_65", 3, 128, (1, 5, 13), 128, 0.95, 8, "bf16"),
    "two_blocks_tail": W("two_blocks_tail", 2, 128, (1, 9, 17), 128, 0.5, 1, "bf16"),
    "p_tiny": W("p_tiny", 2, 64, (3, 8, 16), 64, 1e-6, 0, "bf16"),
    "p_one": W("p_one", 2, 64, (3, 8, 16), 64, 1.0, 0, "bf16"),
    "floor_above_nb": W("floor_above_nb", 2, 64, (2, 8, 16), 64, 0.01, 50, "bf16"),
    "f32_one_token": W("f32_one_token", 2, 32, (1, 1, 1), 16, 0.9, 2, "f32"),
}


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", sorted(CASES))
def test_degenerate_path(name):
    w = CASES[name]
    say(f"edge {name}: {w.heads} heads, grid {w.grid}, d={w.d}, block={w.block}, "
        f"p={w.p}, k={w.k}, {w.dtype}")
    q, k, v, _ = synth.make_inputs(w, DEV)
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, device=DEV)
    out = path.run(q, k, v, w.p, w.k)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    check_gather(path, q, k, range(w.heads))
    check_route(path, w, w.p, range(w.heads), q, k)
    check_schedule(path)
    kvc = path.kv_count.cpu().numpy()
    nb = path.nb
    if w.p >= 1.0 or w.k >= nb:
        assert (kvc == nb).all()
    if w.p < 1e-3 and w.k == 0:
        assert (kvc == 1).all()
    tiles = [(h, i) for h in range(w.heads) for i in range(nb)]
    check_attention(path, w, q, k, v, out, tiles)
    # a second run on the same path object gives the same bytes
    out2 = path.run(q, k, v, w.p, w.k)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


# every MFMA instance of the pair kernel (d, block) through the whole path,
# with a ragged tail and an odd number of q-blocks
SHAPES = [
    ("d64_b128", W("d64_b128", 3, 64, (3, 9, 13), 128, 0.9, 2, "bf16", s_range=(2.0, 64.0))),
    ("d128_b64", W("d128_b64", 3, 128, (3, 9, 13), 64, 0.9, 2, "bf16", s_range=(2.0, 64.0))),
    ("d64_b64", W("d64_b64", 2, 64, (2, 7, 19), 64, 0.85, 3, "bf16", s_range=(2.0, 64.0))),
    ("d128_b128", W("d128_b128", 2, 128, (2, 11, 17), 128, 0.85, 3, "bf16",
                    s_range=(2.0, 64.0))),
]


# tiles of three q-blocks exist for 128-key blocks only
SHAPE_PARAMS = [(name, w, ranks, group) for name, w in SHAPES
                for ranks, group in [(0, None), (2, None), (0, 3), (2, 3)]
                if group is None or w.block == 128]


@pytest.mark.parametrize("name,w,ranks,group", SHAPE_PARAMS,
                         ids=[f"{p[0]}-r{p[2]}-g{p[3] or 2}" for p in SHAPE_PARAMS])
def test_every_mfma_shape(name, w, ranks, group):
    say(f"shape {name}: grid {w.grid}, d={w.d}, block={w.block}, ranks={ranks}, "
        f"group={group}")
    q, k, v, _ = synth.make_inputs(w, DEV)
    kw = dict(ranks=ranks, n_workers=8) if ranks else {}
    if group:
        kw["group"] = group
    path = FVAttnPath(w.heads, w.grid, w.d, w.block, dtype=q.dtype, device=DEV, **kw)
    out = path.run(q, k, v, w.p, w.k)
    torch.cuda.synchronize()
    check_gather(path, q, k, range(w.heads))
    check_route(path, w, w.p, range(w.heads), q, k)
    if not ranks:
        check_schedule(path)
    assert path.group == (group or 2)
    tiles = [(h, i) for h in range(w.heads) for i in range(path.nb)]
    check_attention(path, w, q, k, v, out, tiles)
