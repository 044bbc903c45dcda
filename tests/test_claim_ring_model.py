"""CPU model of the claim ring in the persistent pair attention kernel.

With run-time claims, wave 0 of a workgroup claims tiles ahead and posts
their list positions in a four-slot LDS ring; every wave reads a tile's slot
when the walk opens that tile.  Each walk step runs one union block and has
one workgroup barrier.  An LDS write by one wave is seen by a read in another
wave only if a barrier lies between them: the writer reaches the barrier
after writing, the reader leaves it before reading.

Events sit between barriers.  Step t's part before its barrier lies between
barriers t-1 and t; the part after it, between barriers t and t+1; the
start-up writes come before barrier -1 (the start-up barrier).  Event X in the
interval after barrier a is ordered before event Y in the interval after
barrier b, in another wave, iff a + 1 <= b.

The walk opens tile k+1 before the barrier of the step that runs tile k's
last union block.  The protocol in the kernel posts the slot of tile k+2
after the barrier of the step that opens tile k (slots 0-2 before the
start-up barrier).  The earlier protocol posted it after the barrier of tile
k's first step, which this model shows is unordered when tiles k and k+1 each
have a single union block.
"""
import numpy as np
import pytest

RING = 4
LOOKAHEAD = 2          # tiles claimed beyond the one being opened


def _walk(blocks_per_tile):
    """Step index of each tile's first and last union block."""
    first, last, t = [], [], 0
    for b in blocks_per_tile:
        assert b >= 1
        first.append(t)
        t += b
        last.append(t - 1)
    return first, last


def _events(blocks_per_tile, protocol):
    """Interval index (barrier just before the event) of each tile's slot write
    and slot read."""
    first, last = _walk(blocks_per_tile)
    T = len(blocks_per_tile)
    read = [-1] + [last[k - 1] - 1 for k in range(1, T)]     # tile 0: after the start-up barrier
    write = []
    for k in range(T):
        if protocol == "open_step":
            # slots 0..2 at start-up; tile k >= 3 in the step that opened tile k-2
            write.append(-2 if k <= LOOKAHEAD else last[k - LOOKAHEAD - 1])
        else:   # "first_step": slots 0, 1 at start-up; tile k >= 2 after tile k-2's first barrier
            write.append(-2 if k < LOOKAHEAD else first[k - LOOKAHEAD])
    return write, read


def _ordered(a, b):
    return a + 1 <= b


def _violations(blocks_per_tile, protocol):
    write, read = _events(blocks_per_tile, protocol)
    bad = []
    for k in range(len(blocks_per_tile)):
        if not _ordered(write[k], read[k]):
            bad.append(("read before write", k))
        prev = k - RING                      # the slot's previous tile
        if prev >= 0 and not _ordered(read[prev], write[k]):
            bad.append(("write before previous read", k))
    return bad


def test_first_step_protocol_races_on_single_block_tiles():
    # two consecutive single-block tiles: the slot of tile 2 is read at the
    # step where it is written, with no barrier between
    assert ("read before write", 2) in _violations([1, 1, 1], "first_step")
    assert _violations([2, 2, 2, 2, 2], "first_step") == []
    assert ("read before write", 3) in _violations([3, 1, 1, 2], "first_step")


@pytest.mark.parametrize("seed", range(40))
def test_open_step_protocol_is_ordered(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 60))
    hi = [2, 3, 8, 600][seed % 4]
    blocks = rng.integers(1, hi, size=T).tolist()
    assert _violations(blocks, "open_step") == []


def test_open_step_protocol_all_single_block():
    assert _violations([1] * 100, "open_step") == []
    assert _violations([1, 5] * 20 + [1] * 9, "open_step") == []
