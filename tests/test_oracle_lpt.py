"""Pins for the oracle's LPT work list (CPU only).

The single-GPU schedule is a reading of the pages' load-balancing problem
(aixai.ru FVAttn post, "Runtime Load Balancing (RLB)"): Graham's LPT rule
over tiles.  These tests pin it to a hand-worked case and to the classical
guarantees of LPT.
"""
import itertools

import numpy as np
import pytest

from oracle import lpt


def test_hand_example():
    order, off, tiles, loads = lpt.lpt_schedule(np.array([7, 5, 4, 3, 3, 2]), 2)
    assert order.tolist() == [0, 1, 2, 3, 4, 5]
    assert tiles[off[0]:off[1]].tolist() == [0, 3, 5]
    assert tiles[off[1]:off[2]].tolist() == [1, 2, 4]
    assert loads.tolist() == [12, 12]


def test_order_is_cost_desc_then_index():
    order = lpt.lpt_order(np.array([1, 3, 3, 0, 2, 3]))
    assert order.tolist() == [1, 2, 5, 4, 0, 3]


@pytest.mark.parametrize("seed", range(6))
def test_conservation(seed):
    rng = np.random.default_rng(seed)
    costs = rng.integers(0, 50, size=int(rng.integers(1, 300)))
    W = int(rng.integers(1, 40))
    order, off, tiles, loads = lpt.lpt_schedule(costs, W)
    assert sorted(tiles.tolist()) == list(range(costs.shape[0]))
    assert sorted(order.tolist()) == list(range(costs.shape[0]))
    assert loads.sum() == costs.sum()
    for w in range(W):
        assert loads[w] == costs[tiles[off[w]:off[w + 1]]].sum()
    # makespan <= mean + max cost (the last tile placed on the critical worker
    # went to the least-loaded worker)
    assert loads.max() <= costs.sum() / W + costs.max() + 1e-9


def brute_opt(costs, W):
    best = None
    for assign in itertools.product(range(W), repeat=len(costs)):
        loads = [0] * W
        for c, w in zip(costs, assign):
            loads[w] += c
        m = max(loads)
        best = m if best is None else min(best, m)
    return best


@pytest.mark.parametrize("seed", range(10))
def test_graham_bound(seed):
    rng = np.random.default_rng(50 + seed)
    W = int(rng.integers(2, 4))
    costs = rng.integers(1, 20, size=int(rng.integers(W + 1, 9)))
    _, _, _, loads = lpt.lpt_schedule(costs, W)
    opt = brute_opt(costs.tolist(), W)
    assert loads.max() <= (4.0 / 3.0 - 1.0 / (3 * W)) * opt + 1e-9


def test_one_worker_takes_the_order():
    costs = np.array([4, 9, 1, 9, 0])
    order, off, tiles, loads = lpt.lpt_schedule(costs, 1)
    assert tiles.tolist() == order.tolist() == [1, 3, 0, 2, 4]
    assert off.tolist() == [0, 5]
    assert loads.tolist() == [23]


def test_more_workers_than_tiles():
    costs = np.array([2, 5, 5])
    order, off, tiles, loads = lpt.lpt_schedule(costs, 5)
    assert tiles.tolist() == [1, 2, 0]
    assert off.tolist() == [0, 1, 2, 3, 3, 3]
    assert loads.tolist() == [5, 5, 2, 0, 0]


def test_equal_costs_spread_evenly():
    costs = np.full(23, 7)
    _, off, _, loads = lpt.lpt_schedule(costs, 5)
    assert loads.max() - loads.min() <= 7
    assert np.diff(off).tolist() == [5, 5, 5, 4, 4]


@pytest.mark.parametrize("seed", range(4))
def test_tile_order_keeps_the_assignment(seed):
    rng = np.random.default_rng(200 + seed)
    costs = rng.integers(0, 30, size=int(rng.integers(1, 200)))
    W = int(rng.integers(1, 17))
    o1, off1, t1, l1 = lpt.lpt_schedule(costs, W)
    o2, off2, t2, l2 = lpt.lpt_schedule(costs, W, tile_order=True)
    assert (o1 == o2).all() and (off1 == off2).all() and (l1 == l2).all()
    for w in range(W):
        a, b = t1[off1[w]:off1[w + 1]], t2[off2[w]:off2[w + 1]]
        assert sorted(a.tolist()) == b.tolist()


# --- two-level (grouped) LPT ------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_grouped_with_one_group_is_plain_lpt(seed):
    rng = np.random.default_rng(300 + seed)
    H, tph = int(rng.integers(1, 6)), int(rng.integers(1, 40))
    costs = rng.integers(0, 50, size=(H, tph))
    W = int(rng.integers(1, 20))
    for tile_order in (False, True):
        a = lpt.lpt_schedule(costs.reshape(-1), W, tile_order=tile_order)
        b = lpt.lpt_schedule_grouped(costs, W, 1, tile_order=tile_order)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_head_groups_hand_example():
    # loads 9, 7, 6, 5, 2 over 2 groups: 9->0, 7->1, 6->1 (7 < 9), 5->0 (9 < 13),
    # 2->1 (13 < 14)
    assert lpt.head_groups(np.array([6, 9, 2, 7, 5]), 2).tolist() == [1, 0, 1, 1, 0]


def test_grouped_hand_example():
    # 2 heads x 3 tiles, 4 workers in 2 groups (workers 0, 2 | 1, 3)
    costs = np.array([[5, 1, 4],      # head 0, load 10 -> group 0
                      [3, 3, 2]])     # head 1, load 8  -> group 1
    order, off, tiles, loads = lpt.lpt_schedule_grouped(costs, 4, 2)
    # global order: 0(5) 2(4) 3(3) 4(3) 5(2) 1(1)
    assert order.tolist() == [0, 2, 3, 4, 5, 1]
    lists = [tiles[off[w]:off[w + 1]].tolist() for w in range(4)]
    assert lists == [[0], [3, 5], [2, 1], [4]]
    assert loads.tolist() == [5, 5, 5, 3]


@pytest.mark.parametrize("seed", range(6))
def test_grouped_tiles_stay_in_their_group(seed):
    rng = np.random.default_rng(400 + seed)
    H, tph = int(rng.integers(1, 12)), int(rng.integers(1, 30))
    costs = rng.integers(0, 60, size=(H, tph))
    W = int(rng.integers(1, 40))
    X = int(rng.integers(1, 10))
    order, off, tiles, loads = lpt.lpt_schedule_grouped(costs, W, X)
    Xe = min(X, W)
    hg = lpt.head_groups(costs.sum(1), Xe)
    assert sorted(tiles.tolist()) == list(range(H * tph))
    assert loads.sum() == costs.sum()
    for w in range(W):
        mine = tiles[off[w]:off[w + 1]]
        assert loads[w] == costs.reshape(-1)[mine].sum()
        assert all(hg[t // tph] == w % Xe for t in mine)
    # inside a group the greedy keeps the LPT bound: makespan <= mean + max
    for x in range(Xe):
        ws = np.arange(x, W, Xe)
        tl = np.concatenate([tiles[off[w]:off[w + 1]] for w in ws])
        if tl.size:
            c = costs.reshape(-1)[tl]
            assert loads[ws].max() <= c.sum() / ws.size + c.max() + 1e-9


def test_grouped_given_head_groups_hand_example():
    # 2 groups, workers 0, 2 (group 0) and 1, 3 (group 1); all three heads
    # forced into group 1 by the given map, so group 0's workers stay empty
    costs = np.array([[5, 1], [4, 2], [3, 3]])
    order, offs, tiles, loads = lpt.lpt_schedule_grouped(costs, 4, 2, head_group=[1, 1, 1])
    # LPT order: t0 (5), t2 (4), t4 (3), t5 (3), t3 (2), t1 (1); each to the
    # less-loaded of workers 1 and 3
    assert order.tolist() == [0, 2, 4, 5, 3, 1]
    assert loads.tolist() == [0, 9, 0, 9]
    assert offs.tolist() == [0, 0, 3, 3, 6]
    assert tiles.tolist() == [0, 5, 1, 2, 4, 3]


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_given_groups_tiles_stay_in_them(seed):
    rng = np.random.default_rng(seed)
    H, tph, W, X = 7, 5, 12, 4
    costs = rng.integers(0, 20, size=(H, tph))
    hg = rng.integers(0, X, size=H)
    _, offs, tiles, loads = lpt.lpt_schedule_grouped(costs, W, X, head_group=hg)
    for w in range(W):
        for t in tiles[offs[w]:offs[w + 1]]:
            assert hg[t // tph] == w % X
    assert sorted(tiles.tolist()) == list(range(H * tph))
    assert loads.sum() == costs.sum()


# --- tile costs of q-block groups (the pair tiles of the persistent kernel) ---
# A tile of `group` consecutive q-blocks of one head costs the kept blocks of
# its q-blocks (the load unit is one sparse block: aixai.ru FVAttn post,
# "Runtime Load Balancing (RLB)").  Worked by hand; nB = 5 is odd, so the last
# pair tile of each head holds one q-block.
_KV_HAND = np.array([[3, 1, 4, 1, 5],
                     [9, 2, 6, 5, 3]])


def test_group_costs_hand_example_odd_tail():
    assert lpt.group_costs(_KV_HAND, 2).tolist() == [4, 5, 5, 11, 11, 3]
    assert lpt.group_costs(_KV_HAND, 3).tolist() == [8, 6, 17, 8]
    # one tile per head: the head's whole load
    assert lpt.group_costs(_KV_HAND, 5).tolist() == [14, 25]
    assert lpt.group_costs(_KV_HAND, 9).tolist() == [14, 25]


def test_group_costs_one_is_identity():
    rng = np.random.default_rng(3)
    kv = rng.integers(0, 50, size=(4, 7))
    assert lpt.group_costs(kv, 1).tolist() == kv.reshape(-1).tolist()


@pytest.mark.parametrize("nb,group", [(1, 2), (2, 2), (7, 2), (591, 2), (10, 3), (11, 4)])
def test_group_costs_shape_and_conservation(nb, group):
    rng = np.random.default_rng(nb * 10 + group)
    kv = rng.integers(0, nb + 1, size=(3, nb))
    c = lpt.group_costs(kv, group).reshape(3, -1)
    assert c.shape == (3, -(-nb // group))
    assert c.sum(axis=1).tolist() == kv.sum(axis=1).tolist()
    # the last tile holds the nb % group tail (or a full group)
    tail = nb - (c.shape[1] - 1) * group
    assert c[:, -1].tolist() == kv[:, nb - tail:].sum(axis=1).tolist()
