"""Pins for the oracle's routing (pool, scores, softmax, Top-p + Top-k cut).

The pages fix: per query block, key blocks are kept in order of importance
until the accumulated importance reaches p (aixai.ru FVAttn post, "Top-p vs
Top-k"), at least the k most important blocks are kept (PaperDaily FVAttn
article, method section), and importance comes from pooled Q/K (same
article).  The score formula is a reading (softmax of pooled dot products).
"""
import itertools
import math

import numpy as np
import pytest

from oracle import route as rt


def test_block_sizes_ragged():
    assert rt.block_sizes(105, 16).tolist() == [16] * 6 + [9]
    assert rt.block_sizes(128, 16).tolist() == [16] * 8
    assert rt.num_blocks(75600, 128) == 591
    assert rt.block_sizes(75600, 128)[-1] == 80
    assert rt.block_sizes(147600, 128)[-1] == 16


def test_pool_is_mean_of_true_rows():
    # row r of head h holds value 10*h + r in every column: block mean is the
    # midpoint of the block's first and last row index.
    H, n, d, B = 2, 105, 4, 16
    x = (10.0 * np.arange(H)[:, None, None]
         + np.arange(n)[None, :, None] + np.zeros((1, 1, d)))
    pooled = rt.pool_blocks(x, B)
    for h in range(H):
        for j in range(7):
            lo, hi = j * B, min(n, (j + 1) * B) - 1
            assert np.allclose(pooled[h, j], 10.0 * h + (lo + hi) / 2.0)


def test_pool_divides_by_true_count_not_block_size():
    x = np.ones((1, 20, 2))
    assert np.allclose(rt.pool_blocks(x, 16), 1.0)


def test_scores_hand_example():
    qbar = np.array([[[1.0, 0.0], [0.0, 2.0]]])
    kbar = np.array([[[3.0, 4.0], [1.0, 1.0]]])
    z = rt.block_scores(qbar, kbar)
    assert np.allclose(z[0], np.array([[3.0, 1.0], [8.0, 2.0]]) / math.sqrt(2))


def test_softmax_values_and_invariants():
    P = rt.row_softmax(np.array([[0.0, math.log(3.0)]]))
    assert np.allclose(P, [[0.25, 0.75]])
    rng = np.random.default_rng(0)
    z = rng.normal(size=(3, 5, 7)) * 4
    P = rt.row_softmax(z)
    assert np.allclose(P.sum(-1), 1.0)
    assert np.allclose(rt.row_softmax(z + 123.0), P)
    assert (P > 0).all()


def uniform_row(nb):
    return np.full(nb, 1.0 / nb)


@pytest.mark.parametrize("p,k,expect", [
    (0.5, 0, [0, 1, 2, 3]),
    (0.3, 2, [0, 1, 2]),
    (0.1, 2, [0, 1]),        # the floor is active
    (0.1, 0, [0]),
    (1.0, 0, list(range(8))),
    (1.5, 0, list(range(8))),
    (0.2, 20, list(range(8))),  # k beyond nB keeps everything
])
def test_uniform_row_closed_forms(p, k, expect):
    kept, _, _ = rt.select_row(uniform_row(8), p, k)
    assert kept.tolist() == expect


def test_zero_queries_give_uniform_rows():
    rng = np.random.default_rng(1)
    H, n, d, B = 2, 8 * 16, 8, 16
    q = np.zeros((H, n, d))
    k = rng.normal(size=(H, n, d))
    out = rt.route(q, k, B, 0.5, 0)
    assert np.allclose(out["P"], 1.0 / 8)
    assert (out["kv_count"] == 4).all()
    assert (out["kv_index"][:, :, :4] == np.arange(4)).all()


def test_dominant_block():
    H, nb, B, d = 1, 6, 4, 8
    n = nb * B
    jstar = 4
    q = np.ones((H, n, d)) * 3.0
    k = np.zeros((H, n, d))
    k[:, jstar * B:(jstar + 1) * B, :] = 3.0
    out = rt.route(q, k, B, 0.5, 1)
    assert out["kv_count"].tolist() == [[1] * nb]
    assert (out["kv_index"][0, :, 0] == jstar).all()
    out = rt.route(q, k, B, 0.5, 3)
    for i in range(nb):
        assert out["kv_index"][0, i, :3].tolist() == [0, 1, 4]


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_minimal_prefix(seed):
    """n_p equals the smallest size of ANY subset whose mass reaches p."""
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(2, 11))
    P = rng.dirichlet(np.full(nb, float(rng.uniform(0.2, 3.0))))
    p = float(rng.uniform(0.05, 0.99))
    kept, n_p, _ = rt.select_row(P, p, 0)
    best = nb
    for size in range(1, nb + 1):
        if any(P[list(c)].sum() >= p for c in itertools.combinations(range(nb), size)):
            best = size
            break
    assert n_p == best
    assert P[kept].sum() >= p or n_p == nb


@pytest.mark.parametrize("seed", range(8))
def test_row_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(1, 40))
    k = int(rng.integers(0, 6))
    p = float(rng.uniform(0.05, 1.0))
    P = rng.dirichlet(np.full(nb, float(rng.uniform(0.1, 5.0))))
    kept, n_p, order = rt.select_row(P, p, k)
    S = set(kept.tolist())
    assert len(S) >= min(k, nb)                       # floor
    assert (np.diff(kept) > 0).all()                  # ascending, unique
    if n_p < nb:
        assert P[kept].sum() >= p                     # reaches p
    if len(S) > k and len(S) > 1:                     # minimality of the cut
        weakest = order[len(S) - 1]
        assert P[kept].sum() - P[weakest] < p
    outside = [j for j in range(nb) if j not in S]
    if outside:                                       # top set
        assert P[kept].min() >= P[outside].max()


def test_ties_go_to_lower_index():
    P = np.array([0.2, 0.3, 0.2, 0.3])
    kept, n_p, order = rt.select_row(P, 0.7, 0)
    assert order.tolist() == [1, 3, 0, 2]
    assert kept.tolist() == [0, 1, 3]


def test_route_outputs_and_density():
    rng = np.random.default_rng(3)
    H, n, d, B = 3, 105, 16, 16
    q = rng.normal(size=(H, n, d))
    k = rng.normal(size=(H, n, d))
    out = rt.route(q, k, B, 0.6, 2)
    nb = 7
    assert out["mask"].shape == (H, nb, nb)
    assert (out["mask"].sum(-1) == out["kv_count"]).all()
    for h in range(H):
        for i in range(nb):
            c = out["kv_count"][h, i]
            assert np.flatnonzero(out["mask"][h, i]).tolist() == \
                out["kv_index"][h, i, :c].tolist()
    assert (out["head_load"] == out["kv_count"].sum(-1)).all()
    assert np.allclose(out["head_density"], out["head_load"] / nb ** 2)
    dense = rt.route(q, k, B, 1.0, 0)
    assert (dense["head_density"] == 1.0).all()
    assert (dense["kv_count"] == nb).all()


def test_invalid_arguments():
    q = np.zeros((1, 16, 4))
    with pytest.raises(ValueError):
        rt.route(q, q, 16, 0.0, 1)
    with pytest.raises(ValueError):
        rt.route(q, q, 16, 0.5, -1)
