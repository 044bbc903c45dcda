"""Comparison helpers for the GPU-vs-oracle parity tests.

Mask protocol.  Routing decides integers (which blocks are kept) from
floating-point importances; the GPU computes them in fp32, the oracle in
float64, so rows whose decision sits on a knife edge may legitimately differ.
A row of the GPU mask that differs from the oracle's is accepted only if the
GPU's kept set S is itself a correct answer for the oracle's importances P
within these windows:
  (a) count window: the accumulated mass at the cut is within MASS_WINDOW
      (1e-4) of p, i.e. mass(S) >= p - 1e-4 (at the Top-k floor as well) and,
      when |S| > k, the mass without S's weakest block is < p + 1e-4;
  (b) order window (a reading beyond the stated count window, for rows whose
      importances are nearly uniform): every block in the symmetric
      difference has P within TIE_REL (1e-5) * max P of the cut value, so S is
      a top set up to near-ties.
Every other mismatch fails.  Rows are reported as exact / count / order /
unexplained.
"""
from __future__ import annotations

import numpy as np

MASS_WINDOW = 1e-4
TIE_REL = 1e-5


def classify_rows(P, p, k, gpu_count, gpu_index, ora_count, ora_index):
    """Classify every (h, i) row.  Returns a dict of counts and the list of
    unexplained rows."""
    H, nb, _ = P.shape
    stats = {"rows": H * nb, "exact": 0, "count": 0, "order": 0, "unexplained": 0}
    bad = []
    for h in range(H):
        for i in range(nb):
            gs = gpu_index[h, i, :gpu_count[h, i]]
            os_ = ora_index[h, i, :ora_count[h, i]]
            if gpu_count[h, i] == ora_count[h, i] and np.array_equal(gs, os_):
                stats["exact"] += 1
                continue
            kind = _accept(P[h, i], p, k, gs, os_)
            if kind is None:
                stats["unexplained"] += 1
                bad.append((h, i))
            else:
                stats[kind] += 1
    return stats, bad


def _accept(Prow, p, k, gs, os_):
    nb = Prow.shape[0]
    gs = np.asarray(gs, dtype=np.int64)
    if gs.size == 0 or len(np.unique(gs)) != gs.size or gs.min() < 0 or gs.max() >= nb:
        return None
    if not np.all(np.diff(gs) > 0):
        return None
    if gs.size < min(k, nb):
        return None
    inside = np.zeros(nb, dtype=bool)
    inside[gs] = True
    pin = Prow[inside]
    pout = Prow[~inside]
    tie = TIE_REL * Prow.max()
    # S must be a top set up to near-ties
    if pout.size and pin.min() < pout.max() - tie:
        return None
    mass = pin.sum()
    if p < 1.0:
        # the kept mass reaches p (a row at the Top-k floor too: the floor
        # only wins when the top k already reach p) ...
        if mass < p - MASS_WINDOW:
            return None
        # ... and, above the floor, no smaller prefix would
        if gs.size > k and mass - pin.min() >= p + MASS_WINDOW:
            return None
    elif gs.size != nb:
        return None
    return "count" if gs.size != len(os_) else "order"


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def attn_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    return {"max_abs": float(diff.max()), "rel_l2": rel_l2(got, ref),
            "max_abs_rel": float(diff.max() / max(np.abs(ref).max(), 1e-300))}


# tolerances from the target: max-abs 2e-2 (bf16) / 1e-4 (fp32); relative L2
# added so an all-zero output cannot pass on flat heads with tiny outputs.
TOL = {"bf16": {"max_abs": 2e-2, "rel_l2": 1e-2},
       "f32": {"max_abs": 1e-4, "rel_l2": 1e-5}}
