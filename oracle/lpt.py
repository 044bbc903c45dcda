"""Oracle step 6: longest-processing-time-first (LPT) work list over tiles.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: once the mask exists each head's load (kept sparse blocks
times the time per block) is known exactly, and the aim is to shorten the
critical path left by a few heavy heads (aixai.ru FVAttn post, section
"Runtime Load Balancing (RLB)"; PaperDaily FVAttn article, method section,
where heavy heads are moved greedily from the busiest to the idlest rank).
The pages balance heads across GPU ranks; on one GPU the same problem is the
spread of (head, q-block) tiles over the persistent workgroups.  The pages do
not describe this single-GPU schedule: it is a reading.

Reading taken:
  * tile t = h * nB + i has cost c_t = kv_count[h, i] (kept blocks);
  * tiles are ordered by (cost descending, tile id ascending);
  * in that order each tile goes to the worker with the smallest load so far,
    the lowest worker index on ties (Graham's LPT rule), and is appended to
    that worker's list;
  * outputs: the order, per-worker lists concatenated in worker order with
    offsets, and the final per-worker loads.
One schedule is correct per input.

Pins (tests/test_oracle_lpt.py): a hand-worked two-worker example,
conservation, Graham's 4/3 - 1/(3W) bound against the brute-force optimum,
the makespan <= mean + max-cost bound, W = 1 and W >= tiles.

Two-level variant (lpt_schedule_grouped), a reading of the pages' balancing
between ranks mapped onto the XCDs of one GPU: heads are first spread over
X groups of workers (worker w is in group w % X) by the same LPT rule on
head loads, then every tile goes, in the global LPT order, to the
least-loaded worker of its head's group.  Pins: X = 1 gives lpt_schedule
exactly; tiles stay in their head's group; conservation; a hand example.
The head -> group map can also be given (the per-rank image of SASA/RLB,
oracle/sasa.py); the pins then check that tiles stay in the given groups.
"""
from __future__ import annotations

import numpy as np


def lpt_order(costs: np.ndarray) -> np.ndarray:
    costs = np.asarray(costs, dtype=np.int64)
    t = np.arange(costs.shape[0])
    return np.lexsort((t, -costs)).astype(np.int32)


def lpt_schedule(costs: np.ndarray, n_workers: int, tile_order: bool = False):
    """Greedy LPT.  Returns (order, worker_offsets, worker_tiles, worker_load).

    tile_order=True lists each worker's tiles by ascending tile id instead of
    in assignment order (same assignment, same loads)."""
    if n_workers < 1:
        raise ValueError("n_workers must be >= 1")
    costs = np.asarray(costs, dtype=np.int64).reshape(-1)
    order = lpt_order(costs)
    loads = np.zeros(n_workers, dtype=np.int64)
    lists = [[] for _ in range(n_workers)]
    for t in order:
        w = int(np.argmin(loads))          # argmin returns the lowest index on ties
        lists[w].append(int(t))
        loads[w] += costs[t]
    if tile_order:
        lists = [sorted(x) for x in lists]
    sizes = np.array([len(x) for x in lists], dtype=np.int64)
    offsets = np.zeros(n_workers + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(sizes)
    tiles = np.array([t for x in lists for t in x], dtype=np.int32)
    return order, offsets, tiles, loads


def predicted_imbalance(loads: np.ndarray) -> float:
    loads = np.asarray(loads, dtype=np.float64)
    return float(loads.max() / loads.mean()) if loads.mean() > 0 else 1.0


def group_costs(kv_count, group: int) -> np.ndarray:
    """Cost of each tile of `group` consecutive q-blocks of one head: the sum
    of their kept-block counts.  kv_count [H, nB] -> [H * ceil(nB / group)]."""
    kv = np.asarray(kv_count, dtype=np.int64)
    H, nb = kv.shape
    per = (nb + group - 1) // group
    out = np.zeros((H, per), dtype=np.int64)
    for m in range(per):
        out[:, m] = kv[:, m * group:min(nb, (m + 1) * group)].sum(axis=1)
    return out.reshape(-1)


def head_groups(head_loads: np.ndarray, groups: int) -> np.ndarray:
    """LPT of heads over `groups` bins: heads in (load desc, head asc) order,
    each to the least-loaded group (lowest index on ties).  Returns the group
    of every head."""
    loads = np.asarray(head_loads, dtype=np.int64).reshape(-1)
    gl = np.zeros(groups, dtype=np.int64)
    out = np.zeros(loads.shape[0], dtype=np.int32)
    for h in lpt_order(loads):
        x = int(np.argmin(gl))
        out[h] = x
        gl[x] += loads[h]
    return out


def lpt_schedule_grouped(costs_2d, n_workers: int, groups: int, tile_order: bool = False,
                         head_group=None):
    """Two-level LPT.  costs_2d [H, tiles per head]; worker w belongs to group
    w % X with X = min(groups, n_workers).  Heads go to groups by LPT on their
    summed tile costs (or as `head_group` gives them); then each tile, in the
    global (cost desc, id asc) order, goes to the least-loaded worker of its
    head's group (lowest index on ties).  Returns (order, worker_offsets,
    worker_tiles, worker_load) like lpt_schedule."""
    c2 = np.asarray(costs_2d, dtype=np.int64)
    H, tph = c2.shape
    X = max(1, min(int(groups), n_workers))
    if head_group is None:
        hg = head_groups(c2.sum(axis=1), X)
    else:
        hg = np.clip(np.asarray(head_group, dtype=np.int64), 0, X - 1)
    costs = c2.reshape(-1)
    order = lpt_order(costs)
    loads = np.zeros(n_workers, dtype=np.int64)
    members = [np.arange(x, n_workers, X) for x in range(X)]
    lists = [[] for _ in range(n_workers)]
    for t in order:
        ws = members[hg[t // tph]]
        w = int(ws[np.argmin(loads[ws])])        # first minimum = lowest index
        lists[w].append(int(t))
        loads[w] += costs[t]
    if tile_order:
        lists = [sorted(x) for x in lists]
    offsets = np.zeros(n_workers + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(x) for x in lists])
    tiles = np.array([t for x in lists for t in x], dtype=np.int32)
    return order, offsets, tiles, loads
