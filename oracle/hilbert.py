"""Oracle step 1: Hilbert-curve order of the spatio-temporal token grid.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: tokens are regrouped along a Hilbert curve so that tokens
that are close in space fall into the same or neighbouring blocks, at several
scales (aixai.ru FVAttn post, section "Sparse-routing frontend"; PaperDaily
FVAttn article, method section, where the Hilbert block organisation precedes
routing).  The pages name neither the dimension, the curve variant, the axis
order nor how a grid that is not a power-of-two cube is handled.

Reading taken here (recorded with the other readings in the design notes):
  * one 3D curve over (t, y, x), the whole spatio-temporal grid;
  * the curve is J. Skilling's construction ("Programming the Hilbert curve",
    AIP Conf. Proc. 707, 2004): coordinates are turned into the "transposed"
    index by undoing the excess rotations level by level and Gray-encoding,
    and the index is read by interleaving the transposed words MSB first with
    axis 0 = t, axis 1 = y, axis 2 = x;
  * the curve lives on the enclosing cube of side 2**b,
    b = max(1, ceil(log2(max(T, Y, X)))); grid points are ordered by their
    index on it (all indices are distinct, so there are no ties);
  * token n = (t * Y + y) * X + x (row-major, t slowest).

Pins (tests/test_oracle_hilbert.py): forward/inverse round trip on every point
of the cube for b = 1..4; unit steps along the whole curve; nesting of aligned
runs of 8**m indices into aligned sub-cubes; the b = 1 corner order against a
hand-derived fixture (reflected Gray code); perm/inv_perm bijection.
"""
from __future__ import annotations

import numpy as np

NDIM = 3


def bits_for_grid(T: int, Y: int, X: int) -> int:
    """Bits per axis of the enclosing cube: smallest b >= 1 with 2**b >= max dim."""
    m = max(T, Y, X)
    b = 1
    while (1 << b) < m:
        b += 1
    return b


def axes_to_transpose(coords: np.ndarray, b: int) -> np.ndarray:
    """Skilling's forward step, vectorised over points.

    coords: int64 array [P, 3] of axis values in [0, 2**b).  Returns the
    transposed Hilbert index [P, 3] (bit q of word i is index bit 3*q + (2-i)).
    """
    X = np.array(coords, dtype=np.int64, copy=True)
    n = X.shape[1]
    top = 1 << (b - 1)
    # Undo the excess work, from the top level down.  At level Q the low
    # bits (Q - 1) of every axis are reflected (when that axis' bit Q is set)
    # or exchanged with axis 0 (when it is clear).
    Q = top
    while Q > 1:
        low = Q - 1
        for i in range(n):
            bit_set = (X[:, i] & Q) != 0
            # reflect axis 0's low bits where axis i has bit Q set
            X[bit_set, 0] ^= low
            # exchange the low bits of axis 0 and axis i where it is clear
            clear = ~bit_set
            swap = (X[clear, 0] ^ X[clear, i]) & low
            X[clear, 0] ^= swap
            X[clear, i] ^= swap
        Q >>= 1
    # Gray encode across the axes.
    for i in range(1, n):
        X[:, i] ^= X[:, i - 1]
    fix = np.zeros(X.shape[0], dtype=np.int64)
    Q = top
    while Q > 1:
        fix[(X[:, n - 1] & Q) != 0] ^= Q - 1
        Q >>= 1
    X ^= fix[:, None]
    return X


def transpose_to_axes(T_idx: np.ndarray, b: int) -> np.ndarray:
    """Skilling's inverse step: transposed index [P, 3] -> coordinates [P, 3]."""
    X = np.array(T_idx, dtype=np.int64, copy=True)
    n = X.shape[1]
    # Gray decode.
    t = X[:, n - 1] >> 1
    for i in range(n - 1, 0, -1):
        X[:, i] ^= X[:, i - 1]
    X[:, 0] ^= t
    # Redo the excess work, from the bottom level up, axes in reverse order.
    Q = 2
    limit = 1 << b
    while Q != limit:
        low = Q - 1
        for i in range(n - 1, -1, -1):
            bit_set = (X[:, i] & Q) != 0
            X[bit_set, 0] ^= low
            clear = ~bit_set
            swap = (X[clear, 0] ^ X[clear, i]) & low
            X[clear, 0] ^= swap
            X[clear, i] ^= swap
        Q <<= 1
    return X


def transpose_to_index(T_idx: np.ndarray, b: int) -> np.ndarray:
    """Interleave the transposed words MSB first: axis 0 supplies the top bit."""
    n = T_idx.shape[1]
    h = np.zeros(T_idx.shape[0], dtype=np.int64)
    for q in range(b - 1, -1, -1):
        for i in range(n):
            h = (h << 1) | ((T_idx[:, i] >> q) & 1)
    return h


def index_to_transpose(h: np.ndarray, b: int, n: int = NDIM) -> np.ndarray:
    """Inverse of transpose_to_index."""
    h = np.asarray(h, dtype=np.int64)
    out = np.zeros((h.shape[0], n), dtype=np.int64)
    pos = n * b - 1
    for q in range(b - 1, -1, -1):
        for i in range(n):
            out[:, i] |= ((h >> pos) & 1) << q
            pos -= 1
    return out


def hilbert_index(coords: np.ndarray, b: int) -> np.ndarray:
    """Hilbert index of each point (coords [P, 3] with axis order t, y, x)."""
    return transpose_to_index(axes_to_transpose(coords, b), b)


def hilbert_point(h: np.ndarray, b: int) -> np.ndarray:
    """Point [P, 3] at each Hilbert index."""
    return transpose_to_axes(index_to_transpose(h, b), b)


def grid_coords(T: int, Y: int, X: int) -> np.ndarray:
    """(t, y, x) of token n = (t*Y + y)*X + x, for n = 0..T*Y*X-1."""
    n = np.arange(T * Y * X, dtype=np.int64)
    x = n % X
    y = (n // X) % Y
    t = n // (X * Y)
    return np.stack([t, y, x], axis=1)


def hilbert_order(T: int, Y: int, X: int):
    """perm[r] = token at Hilbert rank r; inv_perm[perm[r]] = r.  int32 each."""
    b = bits_for_grid(T, Y, X)
    keys = hilbert_index(grid_coords(T, Y, X), b)
    perm = np.argsort(keys, kind="stable").astype(np.int32)
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return perm, inv_perm
