"""The C-ABI library: it loads, exports what include/fvattn.h declares, and its
host-side argument validation returns the documented status codes before any
HIP call (so no GPU is needed).  The validation calls run in a subprocess
that sees no GPU, so a validation bug can never launch a kernel on a real
device with the placeholder pointers used here."""
import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_attention_11_amd import _lib  # noqa: E402


def test_library_is_built_in_tree():
    assert os.path.exists(_lib.LIB_PATH), "run __graft_entry__.build() first"
    assert os.path.dirname(_lib.LIB_PATH) == os.path.join(ROOT, "block_sparse_attention_11_amd")


def test_exports_every_declared_symbol():
    lib = _lib.load_library()
    declared = _lib.declared_symbols()
    assert len(declared) == 18, declared
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared) <= exported
    assert set(declared) == set(_lib._SIGNATURES)


def test_version_and_status_strings():
    lib = _lib.load_library()
    assert lib.fvattn_version() == 10000
    assert _lib.status_string(0) == "ok"
    assert _lib.status_string(-1) == "invalid argument"
    assert _lib.status_string(-4) == "workspace missing or too small"
    assert _lib.status_string(-5) == (
        "problem larger than the static scratch of the no-allocation call")
    assert _lib.status_string(7) == "unknown status"


def test_workspace_sizes():
    lib = _lib.load_library()
    # 720p: two pooled fp32 tables [40, 591, 128] and a score table [40, 591, 591]
    pooled = 40 * 591 * 128 * 4
    scores = 40 * 591 * 591 * 4
    rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert lib.fvattn_route_workspace_size(40, 75600, 128, 128) == 2 * rnd(pooled) + rnd(scores)
    assert lib.fvattn_route_workspace_size(0, 75600, 128, 128) == 0
    # ten per-tile slabs plus per-worker counts (up to 2048 workers), group
    # offsets (64 groups + 1) and per-group fallback flags (64 groups)
    assert lib.fvattn_schedule_workspace_size(40, 591, 256) == (
        10 * rnd(40 * 591 * 4) + rnd((2048 + 2 * 64 + 1) * 4))
    assert lib.fvattn_schedule_workspace_size(40, 591, 0) == 0
    # the no-allocation schedule's static scratch takes 40 heads x 4096 q-blocks
    # and refuses 64 x 4096
    assert lib.fvattn_schedule_workspace_size(40, 4096, 2048) <= _lib.NOALLOC_SCRATCH_BYTES
    assert lib.fvattn_schedule_workspace_size(64, 4096, 2048) > _lib.NOALLOC_SCRATCH_BYTES
    # SASA: row stats (float2) + 256-bin histograms + group state (16 B) +
    # per-row tie counts (int32) and offsets (int64)
    rows = 40 * 591
    assert lib.fvattn_sasa_workspace_size(40, 75600, 128, 8) == (
        rnd(8 * rows) + rnd(4 * 256 * 8) + rnd(16 * 8) + rnd(4 * rows) + rnd(8 * rows))
    assert lib.fvattn_sasa_workspace_size(40, 75600, 128, 0) == 0


def _validation_main():
    """Runs in a child process with no visible GPU."""
    lib = _lib.load_library()
    P = ctypes.c_void_p(4096)      # placeholder, never dereferenced
    Q = ctypes.c_void_p(8192)      # a second one, where two must differ
    N = None
    EINVAL, EUNS, EWS = _lib.EINVAL, _lib.EUNSUPPORTED, _lib.EWORKSPACE
    checks = [
        # hilbert
        (lib.fvattn_hilbert_permute(2, 8, 8, N, P, N), EINVAL),
        (lib.fvattn_hilbert_permute(0, 8, 8, P, P, N), EINVAL),
        (lib.fvattn_hilbert_permute(2, 1025, 8, P, P, N), EINVAL),
        # permute
        (lib.fvattn_permute_rows(P, P, P, 1, 16, 8, 1, N), EINVAL),   # src == dst
        (lib.fvattn_permute_rows(P, ctypes.c_void_p(8192), P, 1, 16, 8, 7, N), EINVAL),
        (lib.fvattn_permute_rows(P, ctypes.c_void_p(8192), N, 1, 16, 8, 1, N), EINVAL),
        # route
        (lib.fvattn_route(P, P, 1, 1, 128, 64, 16, 0.0, 2, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route(P, P, 1, 1, 128, 64, 16, -0.5, 2, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route(P, P, 1, 1, 128, 64, 16, float("nan"), 2, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route(P, P, 1, 1, 128, 64, 16, 0.9, -1, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route(P, P, 1, 1, 128, 64, 16, 0.9, 2, N, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route(P, P, 1, 1, 128, 264, 16, 0.9, 2, P, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_route(P, P, 1, 1, 128, 60, 16, 0.9, 2, P, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_route(P, P, 1, 1, 4097 * 16, 64, 16, 0.9, 2, P, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_route(P, P, 1, 1, 128, 64, 16, 0.9, 2, P, P, P, P, P, N, 1 << 30, N), EWS),
        (lib.fvattn_route(P, P, 1, 1, 128, 64, 16, 0.9, 2, P, P, P, P, P, P, 16, N), EWS),
        # permute + pool
        (lib.fvattn_permute_pool(P, P, P, 1, 128, 64, 16, 1, P, N), EINVAL),    # src == dst
        (lib.fvattn_permute_pool(P, Q, P, 1, 128, 64, 16, 1, N, N), EINVAL),    # no pooled
        (lib.fvattn_permute_pool(P, Q, N, 1, 128, 64, 16, 1, P, N), EINVAL),
        (lib.fvattn_permute_pool(P, Q, P, 1, 128, 64, 16, 7, P, N), EINVAL),    # dtype
        (lib.fvattn_permute_pool(P, Q, P, 1, 128, 64, 0, 1, P, N), EINVAL),
        (lib.fvattn_permute_pool(ctypes.c_void_p(4104), Q, P, 1, 128, 64, 16, 1, P, N),
         EINVAL),                                                               # unaligned
        (lib.fvattn_permute_pool(P, Q, P, 1, 128, 264, 16, 1, P, N), EUNS),     # d > 256
        (lib.fvattn_permute_pool(P, Q, P, 1, 128, 60, 16, 1, P, N), EUNS),      # bf16 d % 8
        (lib.fvattn_permute_pool(P, Q, P, 1, 128, 62, 16, 0, P, N), EUNS),      # f32 d % 4
        # route from pooled means
        (lib.fvattn_route_pooled(P, P, 1, 128, 64, 16, 0.0, 2, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route_pooled(P, P, 1, 128, 64, 16, 0.9, -1, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route_pooled(N, P, 1, 128, 64, 16, 0.9, 2, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route_pooled(P, P, 0, 128, 64, 16, 0.9, 2, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_route_pooled(P, P, 1, 128, 62, 16, 0.9, 2, P, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_route_pooled(P, P, 1, 4097 * 16, 64, 16, 0.9, 2, P, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_route_pooled(P, P, 1, 128, 64, 16, 0.9, 2, P, P, P, P, P, N, 1 << 30, N), EWS),
        (lib.fvattn_route_pooled(P, P, 1, 128, 64, 16, 0.9, 2, P, P, P, P, P, P, 16, N), EWS),
        # schedule
        (lib.fvattn_schedule(P, 40, 591, 1, 2049, 0, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_schedule(P, 40, 591, 1, 256, 2, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule(P, 40, 591, 1, 0, 1, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule(N, 40, 591, 1, 256, 1, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule(P, 40, 591, 1, 256, 1, P, P, P, P, P, 100, N), EWS),
        # two-level LPT: at most 64 groups, no more groups than workers,
        # at most 4096 heads
        (lib.fvattn_schedule(P, 40, 591, 1, 256, 65 << 8, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule(P, 40, 591, 1, 4, 8 << 8, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule(P, 4097, 2, 1, 256, 8 << 8, P, P, P, P, P, 1 << 30, N), EUNS),
        # schedule on the static scratch: same checks, then the 8 MiB limit
        # (checked before any HIP call)
        (lib.fvattn_schedule_noalloc(P, 40, 591, 1, 2049, 0, P, P, P, P, N), EUNS),
        (lib.fvattn_schedule_noalloc(P, 40, 591, 1, 256, 2, P, P, P, P, N), EINVAL),
        (lib.fvattn_schedule_noalloc(N, 40, 591, 1, 256, 0, P, P, P, P, N), EINVAL),
        (lib.fvattn_schedule_noalloc(P, 40, 591, 4, 256, 0, P, P, P, P, N), EINVAL),
        (lib.fvattn_schedule_noalloc(P, 40, 591, 1, 4, 8 << 8, P, P, P, P, N), EINVAL),
        (lib.fvattn_schedule_noalloc(P, 4097, 2, 1, 256, 8 << 8, P, P, P, P, N), EUNS),
        (lib.fvattn_schedule_noalloc(P, 64, 4096, 2, 256, 8 << 8, P, P, P, P, N),
         _lib.ESCRATCH),
        (lib.fvattn_schedule_noalloc(P, 1, 1 << 30, 1, 256, 0, P, P, P, P, N),
         _lib.ESCRATCH),
        # attention
        (lib.fvattn_sparse_attn(P, P, P, N, 1, 1, 128, 64, 16, 0, 1, 0.0, P, P, N, N, 0, N, N, 0, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 3, 1, 128, 64, 16, 0, 1, 0.0, P, P, N, N, 0, N, N, 0, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 256, 16, 0, 1, 0.0, P, P, N, N, 0, N, N, 0, N, N), EUNS),
        # a head of 131072 blocks: its kv lists (nB^2 entries) pass 2^31 and
        # are refused before the 4 GiB per-head bound of the V tiles applies
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, (1 << 24) - 1, 128, 128, 1, 2, 0.0, P, P, N, N, 0, N, N, 0, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 0, 1, float("inf"), P, P, N, N, 0, N, N, 0, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 0, 1, 0.0, P, P, P, N, 4, N, N, 0, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 0, 1, 0.0, P, P, P, P, 0, N, N, 0, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 0, 1, 0.0, P, P, N, N, 0, P, N, 0, N, N), EINVAL),
        # run-time claims need the persistent launch
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 0, 1, 0.0, P, P, N, N, 0, N, P, 0, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 2, 1, 0.0, P, P, N, N, 0, N, N, 0, N, N), EINVAL),
        # workers
        (lib.fvattn_attn_workers(1, 128, 128, 1, 2, N), EINVAL),
        (lib.fvattn_attn_workers(1, 128, 128, 1, 4, ctypes.byref(ctypes.c_int())), EINVAL),
        (lib.fvattn_attn_workers(1, 128, 64, 1, 3, ctypes.byref(ctypes.c_int())), EUNS),
        (lib.fvattn_attn_workers(1, 128, 128, 0, 3, ctypes.byref(ctypes.c_int())), EUNS),
        (lib.fvattn_attn_workers(1, 128, 128, 5, 1, ctypes.byref(ctypes.c_int())), EINVAL),
        (lib.fvattn_schedule(P, 40, 591, 4, 256, 1, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule(P, 40, 591, 0, 256, 1, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 1, 4, 0.0, P, P, N, N, 0, N, N, 0, N, N), EINVAL),
        # three q-blocks per tile: bf16 V tiles of 128-key blocks only
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 1, 3, 0.0, P, P, N, N, 0, N, N, 0, N, N), EUNS),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 256, 128, 128, 0, 3, 0.0, P, P, N, N, 0, N, N, 0, N, N), EUNS),
        (lib.fvattn_sparse_attn(P, P, P, P, 0, 1, 256, 128, 128, 1, 3, 0.0, P, P, N, N, 0, N, N, 0, N, N), EUNS),
        # pack_v
        (lib.fvattn_pack_v(P, P, P, 1, 128, 64, 16, 1, N), EINVAL),
        (lib.fvattn_pack_v(P, ctypes.c_void_p(8192), P, 1, 128, 64, 16, 0, N), EUNS),
        (lib.fvattn_pack_v(P, ctypes.c_void_p(8192), P, 1, 128, 60, 16, 1, N), EUNS),
        (lib.fvattn_pack_v(P, ctypes.c_void_p(8192), P, 1, 128, 64, 18, 1, N), EUNS),
        (lib.fvattn_pack_v(P, ctypes.c_void_p(8192), P, 1, 128, 64, 12, 1, N), EUNS),
        (lib.fvattn_pack_v(P, ctypes.c_void_p(8192), P, 1, 128, 64, 8, 1, N), EUNS),
        (lib.fvattn_pack_v(P, ctypes.c_void_p(8192), P, 1, 128, 64, 24, 1, N), EUNS),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 12, 1, 1, 0.0, P, P, N, N, 0, N, N, 0, N, N), EUNS),
        (lib.fvattn_pack_v(P, ctypes.c_void_p(8192), N, 1, 128, 64, 16, 1, N), EINVAL),
        # claim groups: 0..64
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 0, 1, 0.0, P, P, P, P, 4, N, P, 65, N, N), EINVAL),
        (lib.fvattn_sparse_attn(P, P, P, P, 1, 1, 128, 64, 16, 0, 1, 0.0, P, P, P, P, 4, N, P, -1, N, N), EINVAL),
        # schedule with given head groups
        (lib.fvattn_schedule_heads(P, 40, 591, 1, 256, 8, N, 0, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule_heads(P, 40, 591, 1, 256, 1, P, 0, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule_heads(P, 40, 591, 1, 256, 65, P, 0, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule_heads(P, 40, 591, 1, 4, 8, P, 0, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule_heads(P, 40, 591, 1, 256, 8, P, 8 << 8, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule_heads(P, 40, 591, 4, 256, 8, P, 0, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_schedule_heads(P, 40, 591, 1, 2049, 8, P, 0, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_schedule_heads(P, 40, 591, 1, 256, 8, P, 0, P, P, P, P, P, 100, N), EWS),
        # SASA plan: thresholds and sizes
        (lib.fvattn_sasa_plan(N, 40, 8, 1.05, 1.10, 0.8, 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 0, 8, 1.05, 1.10, 0.8, 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 40, 0, 1.05, 1.10, 0.8, 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 40, 8, 0.95, 1.10, 0.8, 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 40, 8, 1.05, 1.00, 0.8, 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 40, 8, 1.05, float("inf"), 0.8, 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 40, 8, 1.05, 1.10, 1.5, 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 40, 8, 1.05, 1.10, 0.8, -0.1, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 40, 8, 1.05, 1.10, float("nan"), 0.07, P, P, P, N), EINVAL),
        (lib.fvattn_sasa_plan(P, 4097, 8, 1.05, 1.10, 0.8, 0.07, P, P, P, N), EUNS),
        (lib.fvattn_sasa_plan(P, 40, 65, 1.05, 1.10, 0.8, 0.07, P, P, P, N), EUNS),
        # SASA augment
        (lib.fvattn_sasa_augment(N, 1 << 30, 1, 128, 64, 16, P, P, 2, P, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_sasa_augment(P, 1 << 30, 1, 128, 64, 16, P, P, 0, P, P, P, P, P, P, P, 1 << 30, N), EINVAL),
        (lib.fvattn_sasa_augment(P, 1 << 30, 1, 128, 64, 16, P, P, 2, P, P, P, P, P, N, P, 1 << 30, N), EINVAL),
        (lib.fvattn_sasa_augment(P, 1 << 30, 1, 4097 * 16, 64, 16, P, P, 2, P, P, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_sasa_augment(P, 1 << 30, 1, 128, 64, 16, P, P, 65, P, P, P, P, P, P, P, 1 << 30, N), EUNS),
        (lib.fvattn_sasa_augment(P, 16, 1, 128, 64, 16, P, P, 2, P, P, P, P, P, P, P, 1 << 30, N), EWS),
        (lib.fvattn_sasa_augment(P, 1 << 30, 1, 128, 64, 16, P, P, 2, P, P, P, P, P, P, N, 1 << 30, N), EWS),
        (lib.fvattn_sasa_augment(P, 1 << 30, 1, 128, 64, 16, P, P, 2, P, P, P, P, P, P, P, 8, N), EWS),
    ]
    bad = [(i, got, want) for i, (got, want) in enumerate(checks) if got != want]
    if bad:
        print("MISMATCH", bad)
        sys.exit(1)
    print("validation ok", len(checks))


def test_validation_error_codes():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    code = ("import sys; sys.path.insert(0, %r); import tests.test_abi as t; "
            "t._validation_main()" % ROOT)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         env=env, cwd=ROOT, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "validation ok" in res.stdout


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        _lib.hilbert_permute(1, 2, 2, x, x)


def test_header_is_plain_c(tmp_path):
    """include/fvattn.h compiles as C99 (a C caller needs no C++)."""
    src = tmp_path / "use.c"
    src.write_text('#include "fvattn.h"\nint main(void) { return fvattn_version() < 0; }\n')
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                          "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
                          "-I/opt/rocm/include", str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
