"""GPU test of fvattn_schedule_noalloc, the schedule entry point that
allocates nothing (its scratch is the library's static device array).

Through the C ABI it must give fvattn_schedule's outputs bit for bit (the
integer schedule has one correct result per input), on two calls in a row
where the second is smaller (the scratch keeps the first call's contents),
for plain, two-level (8 groups) and tile-ordered lists; a problem larger
than the static scratch is refused before anything is launched.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_11_amd import _lib

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def _kv(heads, nb, seed):
    g = torch.Generator().manual_seed(seed)
    base = torch.randint(1, nb + 1, (heads, 1), generator=g)
    jitter = torch.randint(0, max(2, nb // 8), (heads, nb), generator=g)
    return torch.clamp(base + jitter - nb // 16, 1, nb).to(torch.int32).to(DEV)


def _outputs(heads, nb, group, W):
    tiles = heads * ((nb + group - 1) // group)
    return (torch.full((tiles,), -7, dtype=torch.int32, device=DEV),
            torch.full((W + 1,), -7, dtype=torch.int32, device=DEV),
            torch.full((tiles,), -7, dtype=torch.int32, device=DEV),
            torch.full((W,), -7, dtype=torch.int64, device=DEV))


def _both(kv, W, group, groups, tile_order):
    heads, nb = kv.shape
    ref = _outputs(heads, nb, group, W)
    ws = torch.empty(_lib.schedule_workspace_size(heads, nb, W), dtype=torch.uint8, device=DEV)
    _lib.schedule(kv, W, *ref, ws, tile_order=tile_order, group=group, worker_groups=groups)
    got = _outputs(heads, nb, group, W)
    _lib.schedule_noalloc(kv, W, *got, tile_order=tile_order, group=group,
                          worker_groups=groups)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("groups,tile_order", [(1, False), (8, False), (8, True), (1, True)])
def test_noalloc_schedule_equals_workspace_schedule(groups, tile_order):
    # 1st call: the long 720p shape (40 heads x 1154 q-blocks, pairs, 256
    # workers); 2nd call, smaller: 7 heads x 333 q-blocks (odd), 64 workers
    for heads, nb, group, W, seed in ((40, 1154, 2, 256, 1), (7, 333, 2, 64, 2),
                                      (5, 100, 1, 24, 3)):
        say(f"noalloc schedule {heads}x{nb} group={group} W={W} groups={groups} "
            f"tile_order={tile_order}")
        kv = _kv(heads, nb, seed)
        ref, got = _both(kv, W, group, groups, tile_order)
        for r, g, what in zip(ref, got, ("order", "offsets", "tiles", "loads")):
            assert torch.equal(r, g), what


def test_noalloc_schedule_refuses_oversize():
    kv = torch.ones((64, 4096), dtype=torch.int32, device=DEV)
    out = _outputs(64, 4096, 2, 256)
    with pytest.raises(_lib.FvattnError) as e:
        _lib.schedule_noalloc(kv, 256, *out, group=2, worker_groups=8)
    assert e.value.status == _lib.ESCRATCH
    torch.cuda.synchronize()
    assert (out[0] == -7).all()               # nothing was launched
