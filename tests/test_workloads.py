"""Host logic of the synthetic workloads: shapes, seeds, ragged lengths."""
import math

import numpy as np
import pytest

import workloads as W


def test_uniform_shapes():
    expect = {"tiny": (64, 512, 4), "page_demo": (512, 4096, 8), "shard70b": (2048, 8192, 8), "long128k": (16384, 8192, 8)}
    for name, (T, h, t) in expect.items():
        w = W.BY_NAME[name]
        b, s, TT, cu = W.shard_geometry(w)
        assert (TT, w.h, w.t) == (T, h, t) and cu is None and b * s // t == T


def test_ragged_length_distribution_parameters():
    # The lognormal's arithmetic mean and CV must be the stated 4096 and 0.18.
    w = W.BY_NAME["ragged13b"]
    big = W.Workload(**{**w.__dict__, "nseq": 400_000})
    x = W.ragged_lengths(np.random.default_rng(0), big).astype(np.float64)
    assert abs(x.mean() / 4096 - 1) < 0.003
    assert abs(x.std() / x.mean() - 0.18) < 0.003
    assert np.all(x % 8 == 0) and np.all(x >= 8)


def test_ragged_inputs_small():
    w = W.BY_NAME["ragged13b"]
    inp = W.make_inputs(w, with_dy=False)
    cu = inp["cu_seqlens"]
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0) and cu[-1] == inp["T"]
    assert inp["s"] == int(inp["lengths"].sum()) and inp["T"] * 8 == inp["s"]
    assert inp["partials"].shape == (8, inp["T"], 5120) and inp["partials"].dtype == np.uint16
    assert inp["residual"] is None and inp["bias"] is None and inp["beta"] is None
    assert 3000 < inp["T"] < 5200


def test_deterministic_and_bf16_storage_is_torch_cast():
    import torch
    w = W.BY_NAME["page_demo"]
    a = W.make_inputs(w, with_dy=False)
    b = W.make_inputs(w, with_dy=False)
    assert np.array_equal(a["partials"], b["partials"]) and np.array_equal(a["gamma"], b["gamma"])
    rng = np.random.default_rng(w.input_seed)
    x = (rng.standard_normal((w.b * w.s // w.t, w.h)) * w.slab_scale).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(a["partials"][0], ref)


def test_tiny_is_fp32_with_all_inputs():
    inp = W.make_inputs(W.BY_NAME["tiny"])
    for k in ("residual", "bias", "gamma", "beta", "dy"):
        assert inp[k] is not None and inp[k].dtype == np.float32
    g = inp["gamma"]
    assert g.min() >= 0.5 and g.max() <= 1.5
