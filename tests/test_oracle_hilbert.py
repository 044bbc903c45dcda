"""Pins for the oracle's Hilbert order (CPU only).

The pages fix only that tokens are regrouped along a Hilbert curve so nearby
tokens share or neighbour blocks (aixai.ru FVAttn post, "Sparse-routing
frontend").  The curve is read as Skilling's 3D construction; these tests pin
the oracle to what that construction and a Hilbert curve must satisfy.
"""
import os

import numpy as np
import pytest

from oracle import hilbert as hb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cube_points(b):
    n = 1 << b
    g = np.stack(np.meshgrid(np.arange(n), np.arange(n), np.arange(n),
                             indexing="ij"), -1)
    return g.reshape(-1, 3).astype(np.int64)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_round_trip_every_point(b):
    pts = cube_points(b)
    h = hb.hilbert_index(pts, b)
    assert sorted(h.tolist()) == list(range(8 ** b))        # a bijection
    assert (hb.hilbert_point(h, b) == pts).all()            # exact inverse


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5])
def test_unit_steps(b):
    """Consecutive curve points are face neighbours (L1 distance exactly 1)."""
    pts = hb.hilbert_point(np.arange(8 ** b), b)
    step = np.abs(np.diff(pts, axis=0)).sum(axis=1)
    assert (step == 1).all()
    assert (pts[0] == 0).all()


@pytest.mark.parametrize("b,m", [(2, 1), (3, 1), (3, 2), (4, 2), (4, 3)])
def test_nesting(b, m):
    """Every aligned run of 8**m indices fills one aligned 2**m sub-cube."""
    pts = hb.hilbert_point(np.arange(8 ** b), b)
    side = 1 << m
    for start in range(0, 8 ** b, 8 ** m):
        run = pts[start:start + 8 ** m]
        lo = run.min(axis=0)
        assert (lo % side == 0).all()
        assert (run.max(axis=0) - lo == side - 1).all()
        assert len({tuple(p) for p in run.tolist()}) == 8 ** m


def test_b1_corner_order_matches_hand_derivation():
    rows = np.loadtxt(os.path.join(GOLDEN, "hilbert_b1_corners.txt"),
                      dtype=np.int64, comments="#")
    pts = hb.hilbert_point(rows[:, 0], 1)
    assert (pts == rows[:, 1:]).all()
    assert (hb.hilbert_index(rows[:, 1:], 1) == rows[:, 0]).all()


@pytest.mark.parametrize("grid", [(2, 8, 8), (3, 5, 7), (4, 16, 16),
                                  (1, 1, 1), (1, 1, 5), (21, 45, 80)])
def test_perm_is_bijection_with_exact_inverse(grid):
    perm, inv = hb.hilbert_order(*grid)
    n = grid[0] * grid[1] * grid[2]
    assert perm.dtype == np.int32 and inv.dtype == np.int32
    assert sorted(perm.tolist()) == list(range(n))
    assert (inv[perm] == np.arange(n)).all()
    assert (perm[inv] == np.arange(n)).all()


def test_perm_on_cube_grid_follows_the_curve():
    """On a full 2**b cube the grid order is the curve itself: unit steps."""
    perm, _ = hb.hilbert_order(8, 8, 8)
    coords = hb.grid_coords(8, 8, 8)[perm]
    assert (np.abs(np.diff(coords, axis=0)).sum(axis=1) == 1).all()


def test_perm_orders_tokens_by_their_curve_index():
    grid = (3, 5, 7)
    b = hb.bits_for_grid(*grid)
    perm, _ = hb.hilbert_order(*grid)
    keys = hb.hilbert_index(hb.grid_coords(*grid), b)
    assert (np.diff(keys[perm]) > 0).all()


def test_bits_for_grid():
    assert hb.bits_for_grid(1, 1, 1) == 1
    assert hb.bits_for_grid(2, 2, 2) == 1
    assert hb.bits_for_grid(21, 45, 80) == 7
    assert hb.bits_for_grid(41, 45, 80) == 7
    assert hb.bits_for_grid(3, 5, 129) == 8


def test_token_index_is_t_major():
    c = hb.grid_coords(2, 3, 4)
    assert c[0].tolist() == [0, 0, 0]
    assert c[1].tolist() == [0, 0, 1]
    assert c[4].tolist() == [0, 1, 0]
    assert c[12].tolist() == [1, 0, 0]


def test_locality_blocks_are_compact():
    """Hilbert blocks of 512 tokens on a 16^3 grid are aligned 8^3 cubes,
    whereas row-major blocks span two whole x-rows."""
    perm, _ = hb.hilbert_order(16, 16, 16)
    coords = hb.grid_coords(16, 16, 16)[perm]
    for j in range(8):
        blk = coords[j * 512:(j + 1) * 512]
        assert (blk.max(axis=0) - blk.min(axis=0) == 7).all()
