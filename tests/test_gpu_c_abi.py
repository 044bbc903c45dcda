"""The C ABI used from C alone: tests/c_abi/fvattn_path.c (built by the
build step, linked against libfvattn.so, no Python or torch inside) runs the
whole path and writes its inputs and outputs; here they are checked against
the oracle: the Hilbert order bit for bit, every routed row by the row
protocol, and attention on every tile of the GPU's kept lists."""
import os
import subprocess

import numpy as np
import pytest

from oracle import attention as oat
from oracle import hilbert as ohb
from oracle import route as ort
from tests.parity import TOL, attn_errors, classify_rows

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "fvattn_path")


def read_bf16(path, shape):
    u = np.fromfile(path, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64).reshape(shape)


@pytest.mark.parametrize("grid,heads,d,block,p,kf", [
    ((3, 8, 15), 3, 128, 128, 0.9, 2),       # 360 tokens: two full blocks and a tail
    ((2, 9, 11), 2, 64, 64, 0.8, 1),
])
def test_c_program_whole_path(tmp_path, grid, heads, d, block, p, kf):
    assert os.path.exists(BIN), "run the build step first"
    print(f"C ABI program grid={grid} heads={heads} d={d} block={block}", flush=True)
    res = subprocess.run([BIN, *map(str, grid), str(heads), str(d), str(block), str(p), str(kf),
                          str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    n = grid[0] * grid[1] * grid[2]
    nb = (n + block - 1) // block
    q = read_bf16(tmp_path / "q.bf16", (heads, n, d))
    k = read_bf16(tmp_path / "k.bf16", (heads, n, d))
    v = read_bf16(tmp_path / "v.bf16", (heads, n, d))
    o = read_bf16(tmp_path / "o.bf16", (heads, n, d))
    perm = np.fromfile(tmp_path / "perm.i32", dtype=np.int32)
    gc = np.fromfile(tmp_path / "kv_count.i32", dtype=np.int32).reshape(heads, nb)
    gi = np.fromfile(tmp_path / "kv_index.i32", dtype=np.int32).reshape(heads, nb, nb)
    ref_perm, _ = ohb.hilbert_order(*grid)
    assert np.array_equal(perm, ref_perm)
    qh, kh, vh = (ort.permute_rows(x, perm) for x in (q, k, v))
    ora = ort.route(qh, kh, block, p, kf)
    stats, bad = classify_rows(ora["P"], p, kf, gc, gi, ora["kv_count"], ora["kv_index"])
    assert stats["unexplained"] == 0, bad[:5]
    oh = o[:, perm]                           # O back in Hilbert order
    for h in range(heads):
        for i in range(nb):
            r0, r1 = i * block, min(n, (i + 1) * block)
            ref = oat.block_sparse_attention_tile(qh[h][None], kh[h][None], vh[h][None], 0, i,
                                                  block, gi[h, i, :gc[h, i]])
            err = attn_errors(oh[h, r0:r1], ref)
            assert err["max_abs"] <= TOL["bf16"]["max_abs"] and \
                err["rel_l2"] <= TOL["bf16"]["rel_l2"], (h, i, err)
