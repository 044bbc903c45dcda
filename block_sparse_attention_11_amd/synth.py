"""Seeded synthetic video-shaped Q/K/V workloads.

This module only draws inputs: it holds none of the method's arithmetic and is
shared by the tests, the benchmark and the smoke check, which hand the same
bytes to both the HIP path and the CPU oracle.

Recipe (the pages measure on Wan2.2/2.1 14B activations, which are not
available; these inputs stand in for them at the pages' shapes):
  * grid (T, Y, X) of latent tokens, token n = (t*Y + y)*X + x;
  * per head h a mixing strength s_h and a radius r_h;
  * K, E, V ~ N(0, 1) fp32, drawn in that order per head;
  * Q[h, n] = s_h * mean{K[h, m] : |t_m-t_n|, |y_m-y_n|, |x_m-x_n| <= r_h}
    + E[h, n]  (Chebyshev box clipped at the grid edges, n included; the box
    sums are taken with float64 prefix sums);
  * everything is rounded once to the storage dtype (bf16 with round to
    nearest even, or kept fp32), and those bytes are the single source of
    truth for both sides.
Random numbers: s_h and r_h come from a CPU torch.Generator seeded with the
config's seed (so they do not depend on the device); K, E, V come from a
torch.Generator on the target device seeded with the same seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    d: int
    grid: tuple            # (T, Y, X)
    block: int
    p: float
    k: int
    dtype: str             # "f32" or "bf16"
    s_range: tuple = (0.1, 4.0)      # log-uniform range of s_h
    s_fixed: float | None = None     # overrides s_range for every head
    r_choices: tuple = (1, 2, 3)
    r_fixed: int | None = None
    flat_heads: tuple = ()           # heads forced to s = flat_s
    flat_s: float = 0.1
    seed: int = 0
    note: str = ""

    @property
    def n(self) -> int:
        T, Y, X = self.grid
        return T * Y * X

    @property
    def n_blocks(self) -> int:
        return (self.n + self.block - 1) // self.block

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, (2, 8, 8), 16, 0.9, 2, "f32",
                     s_fixed=1.0, r_fixed=1,
                     note="1 head, d=64, 2x8x8 tokens, block 16, fp32"),
    "small": Workload("small", 8, 64, (4, 16, 16), 64, 0.9, 4, "bf16",
                      note="8 heads, d=64, 4x16x16 tokens, block 64, bf16"),
    "480p": Workload("480p", 40, 128, (21, 30, 52), 128, 0.95, 8, "bf16",
                     note="40 heads, d=128, 21x30x52 tokens, block 128, bf16"),
    "720p": Workload("720p", 40, 128, (21, 45, 80), 128, 0.95, 8, "bf16",
                     flat_heads=tuple(range(32, 40)), flat_s=0.1,
                     note="40 heads, d=128, 21x45x80 tokens, block 128, bf16;"
                          " heads 32-39 flat (s=0.1)"),
    "long720p": Workload("long720p", 40, 128, (41, 45, 80), 128, 0.95, 8, "bf16",
                         note="40 heads, d=128, 41x45x80 tokens, block 128,"
                              " bf16; 4 steps with s_h redrawn per step"),
    # The same long workload at Top-p 0.90 (the pages run both 0.95 and 0.90).
    "long720p_p90": Workload("long720p_p90", 40, 128, (41, 45, 80), 128, 0.90, 8, "bf16",
                             note="40 heads, d=128, 41x45x80 tokens, block 128,"
                                  " bf16, Top-p 0.90; 4 steps with s_h redrawn per step"),
    # Supplementary, labelled: stronger Q/K coupling so routing is really sparse.
    # Routed density per head at this shape (Hilbert blocks, p = 0.95, k = 8):
    # s = 64 -> 0.89-0.92, s = 128 -> 0.54-0.88, s = 256 -> 0.02-0.58,
    # s >= 512 -> near the Top-k floor (8/591), depending on r.
    "720p_sparse": Workload("720p_sparse", 40, 128, (21, 45, 80), 128, 0.95, 8,
                            "bf16", s_range=(64.0, 1024.0),
                            flat_heads=tuple(range(32, 40)), flat_s=64.0,
                            note="supplementary: 720p shape with s_h log-uniform"
                                 " in [64, 1024], heads 32-39 at s=64 (dense, heavy)"),
    # Supplementary, labelled: the long shape with the same strong coupling,
    # s_h (and K, E, V) redrawn every step, so per-head loads move between steps.
    "long720p_sparse": Workload("long720p_sparse", 40, 128, (41, 45, 80), 128, 0.95, 8,
                                "bf16", s_range=(64.0, 1024.0),
                                flat_heads=tuple(range(32, 40)), flat_s=64.0,
                                note="supplementary: long720p shape with s_h log-uniform"
                                     " in [64, 1024] redrawn per step, heads 32-39 at s=64"),
    # One rank's share of the 720p workload under 8-way head sharding.
    "720p_rank": Workload("720p_rank", 5, 128, (21, 45, 80), 128, 0.95, 8, "bf16",
                          note="720p, 5 of 40 heads (one of 8 ranks)"),
}


def _box_sum_axis(x: torch.Tensor, axis: int, r: int) -> torch.Tensor:
    """Sum over a window [i-r, i+r] clipped to the axis, via a prefix sum."""
    L = x.shape[axis]
    c = torch.cumsum(x, dim=axis)
    zero_shape = list(x.shape)
    zero_shape[axis] = 1
    c = torch.cat([torch.zeros(zero_shape, dtype=x.dtype, device=x.device), c],
                  dim=axis)
    idx = torch.arange(L, device=x.device)
    hi = torch.clamp(idx + r, max=L - 1) + 1
    lo = torch.clamp(idx - r, min=0)
    return c.index_select(axis, hi) - c.index_select(axis, lo)


def _box_count_axis(L: int, r: int, device) -> torch.Tensor:
    idx = torch.arange(L, device=device)
    return (torch.clamp(idx + r, max=L - 1) - torch.clamp(idx - r, min=0) + 1
            ).to(torch.float64)


def head_params(w: Workload, seed: int | None = None):
    """(s_h, r_h) lists for a workload, drawn on a CPU generator."""
    seed = w.seed if seed is None else seed
    g = torch.Generator(device="cpu").manual_seed(seed)
    H = w.heads
    u = torch.rand(H, generator=g, dtype=torch.float64)
    lo, hi = w.s_range
    s = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    r = torch.tensor(w.r_choices, dtype=torch.int64)[
        torch.randint(len(w.r_choices), (H,), generator=g)]
    s = s.tolist()
    r = r.tolist()
    if w.s_fixed is not None:
        s = [float(w.s_fixed)] * H
    if w.r_fixed is not None:
        r = [int(w.r_fixed)] * H
    for h in w.flat_heads:
        s[h] = float(w.flat_s)
    return s, r


def make_inputs(w: Workload, device="cpu", seed: int | None = None,
                r_override=None):
    """Draw Q, K, V [H, n, d] in the workload's storage dtype on `device`.

    Returns (q, k, v, meta) with meta = {"s": [...], "r": [...], "seed": ...}.
    `r_override` fixes the radii (the long workload draws them once).
    """
    seed = w.seed if seed is None else seed
    s, r = head_params(w, seed)
    if r_override is not None:
        r = list(r_override)
    T, Y, X = w.grid
    H, n, d = w.heads, w.n, w.d
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.empty((H, n, d), dtype=dt, device=dev)
    k = torch.empty((H, n, d), dtype=dt, device=dev)
    v = torch.empty((H, n, d), dtype=dt, device=dev)
    for h in range(H):
        kh = torch.randn((n, d), generator=g, dtype=torch.float32, device=dev)
        eh = torch.randn((n, d), generator=g, dtype=torch.float32, device=dev)
        vh = torch.randn((n, d), generator=g, dtype=torch.float32, device=dev)
        rr = int(r[h])
        box = kh.to(torch.float64).reshape(T, Y, X, d)
        for axis in range(3):
            box = _box_sum_axis(box, axis, rr)
        cnt = (_box_count_axis(T, rr, dev)[:, None, None]
               * _box_count_axis(Y, rr, dev)[None, :, None]
               * _box_count_axis(X, rr, dev)[None, None, :])
        mean = (box / cnt[..., None]).reshape(n, d)
        qh = (s[h] * mean + eh.to(torch.float64)).to(torch.float32)
        q[h] = qh.to(dt)
        k[h] = kh.to(dt)
        v[h] = vh.to(dt)
        del kh, eh, vh, box, mean, qh
    return q, k, v, {"s": s, "r": r, "seed": seed}


def long_steps(w: Workload, steps: int = 4):
    """Per-step (seed, r) for the long workload: r drawn once, s/K/E/V per step."""
    _, r0 = head_params(w, w.seed)
    return [(st, r0) for st in range(steps)]
