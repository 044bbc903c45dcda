"""Pins for the SASA / RLB oracle (oracle/sasa.py): hand-worked plans for
every mode, RLB moves worked by hand, budgets by hand (with the float64
boundary made explicit), and the augmentation against brute force over all
subsets on tiny tensors."""
import itertools

import numpy as np
import pytest

from oracle import sasa


def test_static_groups_contiguous():
    assert sasa.static_groups(40, 8).tolist() == sum([[g] * 5 for g in range(8)], [])
    # fewer heads than groups: some groups stay empty
    assert sasa.static_groups(5, 8).tolist() == [0, 1, 3, 4, 6]
    assert sasa.static_groups(3, 1).tolist() == [0, 0, 0]


def test_imbalance_and_modes():
    assert sasa.imbalance([10, 10]) == 1.0
    assert sasa.imbalance([30, 10]) == 1.5
    assert sasa.imbalance([0, 0, 0]) == 1.0
    # the three regimes and their closed/open ends
    assert sasa.mode_of(1.0) == sasa.MODE_OFF
    assert sasa.mode_of(1.0499) == sasa.MODE_OFF
    assert sasa.mode_of(1.05) == sasa.MODE_SASA
    assert sasa.mode_of(1.0999) == sasa.MODE_SASA
    assert sasa.mode_of(1.10) == sasa.MODE_RLB_SASA
    assert sasa.mode_of(3.0) == sasa.MODE_RLB_SASA


def test_rlb_heaviest_head_too_heavy_moves_next():
    # groups {0,1} and {2,3}: loads 10 and 2.  Moving head 0 (9) would leave
    # 11 > 10 on the other side, so head 1 (1) moves; group 0 then has given
    # its one head and stays critical.
    grp, moves = sasa.rlb_moves([9, 1, 1, 1], sasa.static_groups(4, 2), 2)
    assert moves == [(1, 0, 1)]
    assert grp.tolist() == [0, 1, 1, 1]
    assert sasa.group_loads([9, 1, 1, 1], grp, 2).tolist() == [9, 3]


def test_rlb_two_moves_by_hand():
    # 3 groups of 2 heads; loads 11, 2, 2.  Move 1: head 0 (6) from group 0
    # to group 1 (2 + 6 < 11) -> 5, 8, 2.  Move 2: group 1 is critical; head 0
    # already moved, head 2 (1) to group 2 (2 + 1 < 8) -> 5, 7, 3.  Group 1
    # has now given a head: stop.
    grp, moves = sasa.rlb_moves([6, 5, 1, 1, 1, 1], sasa.static_groups(6, 3), 3)
    assert moves == [(0, 0, 1), (2, 1, 2)]
    assert grp.tolist() == [1, 0, 2, 1, 2, 2]
    assert sasa.group_loads([6, 5, 1, 1, 1, 1], grp, 3).tolist() == [5, 7, 3]


def test_rlb_balanced_does_nothing():
    grp, moves = sasa.rlb_moves([3, 3, 3, 3], sasa.static_groups(4, 2), 2)
    assert moves == [] and grp.tolist() == [0, 0, 1, 1]


def test_budgets_by_hand():
    # lmax 100: slack 0 -> none; 10 >= 7 -> floor(8.0) = 8; 50 -> 40
    assert sasa.budgets([100, 90, 50]).tolist() == [0, 8, 40]
    # below the trigger: slack 6 < 7
    assert sasa.budgets([100, 94]).tolist() == [0, 0]
    # float64 boundary: 0.07 * 100 rounds to 7.000000000000001, so a slack of
    # exactly 7 does not trigger, and 8 does (floor(0.8 * 8) = 6)
    assert sasa.budgets([100, 93]).tolist() == [0, 0]
    assert sasa.budgets([100, 92]).tolist() == [0, 6]
    assert sasa.budgets([0, 0]).tolist() == [0, 0]


def test_plan_modes():
    # balanced: off, no budget
    p = sasa.plan([10] * 8, 8)
    assert p["mode"] == sasa.MODE_OFF and p["budget"].tolist() == [0] * 8
    # one group 8% heavy: SASA alone (rho = 108*8/(108+7*100) = 1.0693...)
    p = sasa.plan([108] + [100] * 7, 8)
    assert p["mode"] == sasa.MODE_SASA
    assert p["moves"] == [] and p["head_group"].tolist() == list(range(8))
    assert p["budget"].tolist() == [0] + [int(0.8 * 8)] * 7
    # heavy imbalance: RLB then SASA on the balanced loads
    hl = [9, 1, 1, 1]
    p = sasa.plan(hl, 2)
    assert p["mode"] == sasa.MODE_RLB_SASA
    assert p["loads_before"].tolist() == [10, 2]
    assert p["loads_after"].tolist() == [9, 3]
    assert p["budget"].tolist() == [0, int(np.floor(0.8 * 6))]
    assert p["rho_after"] < p["rho_before"]


def _brute_force_augment(P, mask, head_group, budget):
    """All subsets of size b of a group's skipped blocks: keep the one with
    the largest total P; among equal totals the one whose sorted list of
    (h, i, j) comes first."""
    out = mask.copy()
    H = P.shape[0]
    for g, b in enumerate(budget):
        cand = [(h, i, j) for h in range(H) if head_group[h] == g
                for i in range(P.shape[1]) for j in range(P.shape[2]) if mask[h, i, j] == 0]
        b = min(int(b), len(cand))
        if b <= 0:
            continue
        best, best_key = None, None
        for sub in itertools.combinations(cand, b):
            tot = sum(P[x] for x in sub)
            key = (-round(tot, 12), sorted(sub))
            if best_key is None or key < best_key:
                best, best_key = sub, key
        for x in best:
            out[x] = 1
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_augment_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    H, nb = 3, 3
    P = rng.random((H, nb, nb))
    P /= P.sum(-1, keepdims=True)
    mask = (rng.random((H, nb, nb)) < 0.5).astype(np.uint8)
    head_group = np.array([0, 1, 0])
    budget = np.array([3, 2])
    got, added = sasa.augment(P, mask, head_group, budget)
    ref = _brute_force_augment(P, mask, head_group, budget)
    assert np.array_equal(got, ref)
    assert added.tolist() == [int((got - mask)[[0, 2]].sum()), int((got - mask)[1].sum())]


def test_augment_ties_and_overflow():
    # every skipped block has the same P: ties go to (h, i, j) ascending
    P = np.full((2, 2, 2), 0.5)
    mask = np.array([[[1, 0], [0, 0]], [[0, 0], [1, 1]]], dtype=np.uint8)
    got, added = sasa.augment(P, mask, [0, 0], [2])
    assert added.tolist() == [2]
    assert got[0].tolist() == [[1, 1], [1, 0]] and got[1].tolist() == [[0, 0], [1, 1]]
    # a budget larger than the skipped blocks takes them all
    got, added = sasa.augment(P, mask, [0, 0], [100])
    assert added.tolist() == [5] and got.all()


def test_augment_invariants_random():
    rng = np.random.default_rng(7)
    H, nb, G = 6, 7, 3
    P = rng.random((H, nb, nb)) ** 3
    P /= P.sum(-1, keepdims=True)
    mask = (rng.random((H, nb, nb)) < 0.4).astype(np.uint8)
    head_group = np.array([0, 0, 1, 2, 2, 2])
    budget = np.array([5, 0, 9])
    got, added = sasa.augment(P, mask, head_group, budget)
    delta = got.astype(int) - mask.astype(int)
    assert (delta >= 0).all()                      # only additions
    assert delta[2].sum() == 0                     # no budget, no change
    assert added.tolist() == [delta[:2].sum(), 0, delta[3:].sum()]
    assert added.tolist() == [5, 0, 9]
    # top set within each group: every added block is at least as important
    # as every block still skipped
    for g, hs in ((0, [0, 1]), (2, [3, 4, 5])):
        add = P[hs][delta[hs] == 1]
        rest = P[hs][got[hs] == 0]
        assert add.min() >= rest.max()


def test_lists_from_mask():
    mask = np.zeros((1, 3, 3), dtype=np.uint8)
    mask[0, 0, [2, 0]] = 1
    mask[0, 2, 1] = 1
    kc, ki, hl, hd = sasa.lists_from_mask(mask)
    assert kc.tolist() == [[2, 0, 1]]
    assert ki[0, 0, :2].tolist() == [0, 2] and ki[0, 2, 0] == 1 and ki[0, 1, 0] == -1
    assert hl.tolist() == [3] and hd[0] == np.float32(3 / 9)
