"""Oracle for slack-aware sparse augmentation (SASA) and the head moves of
runtime load balancing (RLB), mapped onto the XCD worker groups of one GPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * after balancing, ranks off the critical path wait for it; SASA turns that
    idle time into extra high-value attention blocks on those ranks only, so
    the critical path does not grow (aixai.ru FVAttn post, section
    "Slack-Aware Sparse Augmentation (SASA)"; PaperDaily FVAttn article, SASA
    paragraphs: the budget is each rank's idle time, the extra blocks are
    taken from the blocks the mask skipped, in importance order, and their
    time must not exceed the budget);
  * the routing pass already gives the importance order SASA uses (aixai.ru
    post, section "Sparse-routing frontend");
  * piecewise thresholds on the imbalance factor: k1 = 1.05 and k2 = 1.10;
    SASA alone for k1 <= rho < k2, RLB and then SASA for rho >= k2, nothing
    below k1; an augmentation coefficient n1 = 0.8 and a trigger threshold
    n2 = 0.07 (aixai.ru post, SASA section; PaperDaily article, the layered
    trigger logic);
  * RLB moves at most one local head per rank, heavy heads from overloaded
    to underloaded ranks, when that shortens the critical path (aixai.ru
    post, section "Runtime Load Balancing (RLB)"; PaperDaily article).

Readings taken where the pages are silent or loose (listed in the design
notes):
  * ranks -> the G worker groups of one GPU (worker w in group w % G; G = 8
    XCDs on MI355X); heads start sharded contiguously, head h in group
    floor(h * G / H), as a sequence-parallel split would place them;
  * load of a head = its kept blocks (the routing load); load of a group = the
    sum over its heads; rho = max / mean of the group loads (computed in
    float64);
  * RLB: repeat while the critical group (largest load, lowest index on ties)
    has not yet given a head away: take the least-loaded group (lowest index
    on ties) and move the critical group's heaviest head (lowest index on
    ties) among those not moved before, with load > 0, whose move strictly
    shortens the pair's larger load (load_t + load_h < load_c); stop when no
    such head exists.
    On one GPU a move costs no transfer, so the gain is the critical-path
    reduction alone;
  * SASA budget of group g: slack_g = max load - load_g; the group is
    augmented when slack_g >= n2 * max load, with floor(n1 * slack_g) extra
    blocks (float64);
  * importance of a skipped block (h, i, j) = the routing softmax P[h, i, j];
    a group's extra blocks are its skipped blocks with the largest P,
    ties by (h, i, j) ascending; all of them if the budget is larger.

Pins (tests/test_oracle_sasa.py): hand examples for every mode and for RLB
moves, budgets by hand, brute-force top selection on small tensors,
conservation and invariants (only skipped blocks are added, groups without
budget unchanged, counts equal the budget).
"""
from __future__ import annotations

import math

import numpy as np

K1, K2, N1, N2 = 1.05, 1.10, 0.8, 0.07
MODE_OFF, MODE_SASA, MODE_RLB_SASA = 0, 1, 2


def static_groups(heads: int, groups: int) -> np.ndarray:
    """Contiguous sharding: head h in group floor(h * G / H)."""
    return np.array([h * groups // heads for h in range(heads)], dtype=np.int32)


def group_loads(head_load, head_group, groups: int) -> np.ndarray:
    loads = np.zeros(groups, dtype=np.int64)
    for h, l in enumerate(np.asarray(head_load, dtype=np.int64)):
        loads[int(head_group[h])] += int(l)
    return loads


def imbalance(loads) -> float:
    """rho = max / mean in float64 (1.0 for an all-zero load)."""
    loads = [int(x) for x in loads]
    total = sum(loads)
    if total == 0:
        return 1.0
    return float(max(loads)) * len(loads) / float(total)


def mode_of(rho: float, k1: float = K1, k2: float = K2) -> int:
    if rho < k1:
        return MODE_OFF
    if rho < k2:
        return MODE_SASA
    return MODE_RLB_SASA


def rlb_moves(head_load, head_group, groups: int):
    """Greedy head moves; returns (new head_group, list of (head, from, to))."""
    load_h = [int(x) for x in head_load]
    grp = [int(g) for g in head_group]
    gave = [False] * groups
    moved = [False] * len(grp)
    moves = []
    while True:
        loads = group_loads(load_h, grp, groups)
        c = int(np.argmax(loads))          # first maximum = lowest index on ties
        t = int(np.argmin(loads))
        if gave[c] or c == t:
            break
        cand = sorted((h for h in range(len(grp))
                       if grp[h] == c and load_h[h] > 0 and not moved[h]),
                      key=lambda h: (-load_h[h], h))
        pick = None
        for h in cand:
            if loads[t] + load_h[h] < loads[c]:
                pick = h
                break
        if pick is None:
            break
        grp[pick] = t
        gave[c] = True
        moved[pick] = True
        moves.append((pick, c, t))
    return np.array(grp, dtype=np.int32), moves


def budgets(loads, n1: float = N1, n2: float = N2) -> np.ndarray:
    loads = [int(x) for x in loads]
    lmax = max(loads)
    out = np.zeros(len(loads), dtype=np.int64)
    if lmax <= 0:
        return out
    for g, l in enumerate(loads):
        slack = lmax - l
        if float(slack) >= n2 * float(lmax):
            out[g] = int(math.floor(n1 * float(slack)))
    return out


def plan(head_load, groups: int, k1: float = K1, k2: float = K2, n1: float = N1,
         n2: float = N2):
    """The whole decision: mode, head groups (after RLB when it runs), group
    loads before and after, budgets and the RLB moves."""
    heads = len(head_load)
    grp = static_groups(heads, groups)
    loads0 = group_loads(head_load, grp, groups)
    rho0 = imbalance(loads0)
    mode = mode_of(rho0, k1, k2)
    moves = []
    if mode == MODE_RLB_SASA:
        grp, moves = rlb_moves(head_load, grp, groups)
    loads1 = group_loads(head_load, grp, groups)
    b = budgets(loads1, n1, n2) if mode != MODE_OFF else np.zeros(groups, dtype=np.int64)
    return {"mode": mode, "head_group": grp, "loads_before": loads0, "loads_after": loads1,
            "rho_before": rho0, "rho_after": imbalance(loads1), "budget": b, "moves": moves}


def augment(P: np.ndarray, mask: np.ndarray, head_group, budget):
    """Add, for every group, its budget of skipped blocks with the largest P
    (ties by (h, i, j) ascending).  Returns (new mask, added per group)."""
    P = np.asarray(P, dtype=np.float64)
    H, nb, _ = P.shape
    out = np.array(mask, dtype=np.uint8, copy=True)
    groups = len(budget)
    added = np.zeros(groups, dtype=np.int64)
    for g in range(groups):
        b = int(budget[g])
        if b <= 0:
            continue
        hs = [h for h in range(H) if int(head_group[h]) == g]
        if not hs:
            continue
        cand_h, cand_i, cand_j = [], [], []
        for h in hs:
            ii, jj = np.nonzero(out[h] == 0)
            cand_h.append(np.full(ii.shape, h))
            cand_i.append(ii)
            cand_j.append(jj)
        ch = np.concatenate(cand_h)
        ci = np.concatenate(cand_i)
        cj = np.concatenate(cand_j)
        pv = P[ch, ci, cj]
        order = np.lexsort((cj, ci, ch, -pv))
        take = order[:b]
        out[ch[take], ci[take], cj[take]] = 1
        added[g] = len(take)
    return out, added


def lists_from_mask(mask: np.ndarray):
    """kv_count, kv_index (ascending, -1 padded), head_load, head_density."""
    mask = np.asarray(mask)
    H, nb, _ = mask.shape
    kv_count = mask.sum(-1).astype(np.int32)
    kv_index = np.full((H, nb, nb), -1, dtype=np.int32)
    for h in range(H):
        for i in range(nb):
            idx = np.flatnonzero(mask[h, i])
            kv_index[h, i, :idx.size] = idx
    head_load = kv_count.astype(np.int64).sum(-1)
    head_density = (head_load / float(nb * nb)).astype(np.float32)
    return kv_count, kv_index, head_load, head_density
