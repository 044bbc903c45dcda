"""CPU tests of the mask-row protocol in tests/parity.py: it must accept the
oracle's own answer and the answers the stated windows allow, and reject
every other kept set (a wrong block, a missing floor block, an unsorted or
duplicated list, a set that misses the mass)."""
import numpy as np

from oracle import route as ort
from tests.parity import MASS_WINDOW, TIE_REL, classify_rows


def one_row(P, p, k, gpu_set):
    """Classify one GPU row (kept set gpu_set) against the oracle's answer for
    importance row P."""
    P = np.asarray(P, dtype=np.float64)
    nb = P.shape[0]
    kept, _, _ = ort.select_row(P, p, k)
    ora_count = np.array([[kept.shape[0]]], dtype=np.int32)
    ora_index = np.zeros((1, 1, nb), dtype=np.int32)
    ora_index[0, 0, :kept.shape[0]] = kept
    gc = np.array([[len(gpu_set)]], dtype=np.int32)
    gi = np.zeros((1, 1, nb), dtype=np.int32)
    gi[0, 0, :len(gpu_set)] = gpu_set
    stats, _ = classify_rows(P[None, None, :], p, k, gc, gi, ora_count, ora_index)
    return stats


def test_exact_answer_is_exact():
    P = [0.5, 0.3, 0.15, 0.05]
    s = one_row(P, 0.7, 1, [0, 1])
    assert s["exact"] == 1 and s["unexplained"] == 0


def test_wrong_block_is_rejected():
    P = [0.5, 0.3, 0.15, 0.05]
    assert one_row(P, 0.7, 1, [0, 2])["unexplained"] == 1
    assert one_row(P, 0.7, 1, [1, 3])["unexplained"] == 1


def test_missing_mass_is_rejected():
    P = [0.5, 0.3, 0.15, 0.05]
    assert one_row(P, 0.7, 1, [0])["unexplained"] == 1         # mass 0.5 < 0.7
    assert one_row(P, 0.7, 1, [0, 1, 2])["unexplained"] == 1   # not minimal


def test_floor_is_enforced():
    P = [0.9, 0.05, 0.03, 0.02]
    assert one_row(P, 0.5, 2, [0, 1])["exact"] == 1
    assert one_row(P, 0.5, 2, [0])["unexplained"] == 1


def test_malformed_lists_are_rejected():
    P = [0.4, 0.3, 0.2, 0.1]
    assert one_row(P, 0.6, 1, [1, 0])["unexplained"] == 1       # not ascending
    assert one_row(P, 0.6, 1, [0, 0])["unexplained"] == 1       # duplicate
    assert one_row(P, 0.6, 1, [0, 7])["unexplained"] == 1       # out of range


def test_count_window_accepts_a_cut_on_the_edge():
    # the mass of the top two is p + 1e-5: the oracle keeps 2; a GPU that
    # rounded the prefix sum just below p and kept 3 is inside the window
    P = np.array([0.6, 0.3 + 1e-5, 0.05, 0.05 - 1e-5])
    s = one_row(P, 0.9, 1, [0, 1, 2])
    assert s["count"] == 1 and s["unexplained"] == 0
    # but a cut far from p is not
    P2 = np.array([0.6, 0.35, 0.03, 0.02])
    assert one_row(P2, 0.9, 1, [0, 1, 2])["unexplained"] == 1


def test_order_window_accepts_near_ties_only():
    eps = TIE_REL * 0.25 * 0.1
    P = np.array([0.25 + eps, 0.25, 0.25 - eps, 0.25])
    P = P / P.sum()
    # the oracle keeps the two largest; blocks 1 and 3 tie with block 0's
    # neighbourhood within the relative window
    s = one_row(P, 0.5, 1, [1, 3])
    assert s["unexplained"] == 0
    Q = np.array([0.4, 0.3, 0.2, 0.1])
    assert one_row(Q, 0.6, 1, [0, 2])["unexplained"] == 1


def test_windows_are_the_stated_ones():
    assert MASS_WINDOW == 1e-4 and TIE_REL == 1e-5
