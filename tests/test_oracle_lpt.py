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
