"""The library's host-side batch planning (sp_region_bucket_by_tokens,
sp_region_sp_gate, sp_region_shard_layout, sp_region_cv_within) against the
oracle (oracle/batching.py): integer work, so results must be identical."""
import ctypes
import math

import numpy as np
import pytest

import layernorm_sp_region_amd as spr
import oracle.batching as B
import workloads as W

INVALID = spr.SPR_ERR_INVALID_ARG


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(spr.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return spr.load_library()


def batches(seed=0, count=300):
    rng = np.random.default_rng(seed)
    for k in range(count):
        n = int(rng.integers(0, 80))
        kind = k % 4
        if kind == 0:
            x = rng.integers(0, 9000, n)
        elif kind == 1:
            x = (4096 * rng.lognormal(-0.016, 0.1786, n)).astype(np.int64)   # the ragged workload's mix
        elif kind == 2:
            x = np.where(rng.random(n) < 0.5, rng.integers(50, 200, n), rng.integers(3000, 9000, n))
        else:
            x = rng.choice([0, 1, 2, 4096, 1 << 24], n)
        yield [int(v) for v in x], k


def test_buckets_match_oracle(lib):
    for x, k in batches():
        for cv_bp in (0, 1500, 1800, 5000):
            for budget in (0, 16384, 100000):
                assert spr.bucket_by_tokens(x, cv_bp, budget) == B.bucket_by_tokens(x, cv_bp, budget), (k, cv_bp, budget)


def test_cv_gate_and_layout_match_oracle(lib):
    rng = np.random.default_rng(3)
    for x, k in batches(seed=1, count=200):
        for cv_bp in (0, 900, 1500, 1800, 100000):
            assert spr.cv_within(x, cv_bp) == B.cv_within(x, cv_bp)
        share = float(rng.choice([0.0, 0.1, 0.22, 0.2200001, 0.5]))
        assert spr.sp_gate(x, share) == B.sp_gate(x, share)
        for t in (1, 2, 3, 8):
            assert spr.shard_layout(x, t) == tuple(B.shard_layout(x, t))


def test_ragged_workload_lengths_plan(lib):
    """The 13B-like ragged workload's drawn lengths (CV 0.1798, drawn at the
    page's 0.18) pass the 0.18 gate as one batch and split into two buckets
    at 0.15; the planner's layout of the whole batch is the workload's own."""
    w = W.BY_NAME["ragged13b"]
    lens = W.ragged_lengths(np.random.default_rng(w.input_seed), w)   # the first draw of make_inputs
    lens_l = [int(v) for v in lens]
    order, starts = spr.bucket_by_tokens(lens_l)
    assert (order, starts) == B.bucket_by_tokens(lens_l) and len(starts) == 3
    assert spr.sp_gate(lens_l, 0.0) and not spr.cv_within(lens_l, 1500)
    for a, b in zip(starts, starts[1:]):
        assert spr.cv_within([lens_l[i] for i in order[a:b]], 1500)
    padded, cu, T = spr.shard_layout(lens_l, w.t)
    assert padded == lens_l                        # already multiples of t
    _, _, T_w, cu_w = W.shard_geometry(w, lens)
    assert T == T_w and cu == [int(c) for c in cu_w]


def test_mixed_batch_falls_back_without_buckets(lib):
    """Short and long sequences together exceed the 0.18 gate; each length
    bucket alone passes it (the page's 0.91x -> 0.97x story)."""
    x = [120, 4096, 130, 3900, 125, 4200, 118, 4000]
    assert not spr.sp_gate(x, 0.0)
    order, starts = spr.bucket_by_tokens(x)
    assert len(starts) == 3
    for a, b in zip(starts, starts[1:]):
        assert spr.sp_gate([x[i] for i in order[a:b]], 0.0)


def test_rejects(lib):
    i32 = lambda v: (ctypes.c_int32 * len(v))(*v)
    out = (ctypes.c_int32 * 8)()
    T = ctypes.c_int64()
    ok = i32([5, 6, 7])
    assert lib.sp_region_cv_within(i32([-1, 2]), 2, 100, out) == INVALID
    assert lib.sp_region_cv_within(i32([(1 << 24) + 1]), 1, 100, out) == INVALID
    assert lib.sp_region_cv_within(ok, 3, -1, out) == INVALID
    assert lib.sp_region_cv_within(ok, 3, 100001, out) == INVALID
    assert lib.sp_region_cv_within(ok, 3, 100, None) == INVALID
    assert lib.sp_region_cv_within(None, 3, 100, out) == INVALID
    assert lib.sp_region_cv_within(None, 0, 100, out) == spr.SPR_OK and out[0] == 1
    assert lib.sp_region_bucket_by_tokens(ok, 3, 1500, -1, out, out, out) == INVALID
    assert lib.sp_region_bucket_by_tokens(ok, 3, 1500, 0, None, out, out) == INVALID
    assert lib.sp_region_bucket_by_tokens(ok, 3, 1500, 0, out, out, None) == INVALID
    assert lib.sp_region_sp_gate(ok, 3, math.nan, 1800, 0.22, out) == INVALID
    assert lib.sp_region_sp_gate(ok, 3, 0.1, 1800, math.nan, out) == INVALID
    assert lib.sp_region_shard_layout(ok, 3, 0, out, out, ctypes.byref(T)) == INVALID
    assert lib.sp_region_shard_layout(ok, 3, 9, out, out, ctypes.byref(T)) == INVALID
    assert lib.sp_region_shard_layout(ok, 3, 2, out, out, None) == INVALID
    big = i32([1 << 24] * 200)
    cu = (ctypes.c_int32 * 201)()
    pad = (ctypes.c_int32 * 200)()
    assert lib.sp_region_shard_layout(big, 200, 1, pad, cu, ctypes.byref(T)) == spr.SPR_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        spr.bucket_by_tokens([[1, 2]])
