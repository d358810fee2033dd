"""Pins of the analytic module against the values hpc.payai.win lesson 7 prints
(tests/golden/*.json, each with its citation), closed forms and a simulated ring."""
import json
import os
from fractions import Fraction

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle.analytic import (comm_volume, max_stored_bytes, nontp_activation_bytes, ring_all_gather,
                             ring_reduce_scatter, shape_trace)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_trace_answer_printed_values():
    g = load("lesson7_trace_answer.json")
    i, p = g["inputs"], g["printed"]
    tp_only = shape_trace(i["seq"], i["hidden"], i["tp"], sp=False)
    tp_sp = shape_trace(i["seq"], i["hidden"], i["tp"], sp=True)
    m_tp, m_sp = max_stored_bytes(tp_only), max_stored_bytes(tp_sp)
    assert round(m_tp / 1e6, 1) == p["tp_only_peak_MB"]
    assert round(m_sp / 1e6, 1) == p["tp_sp_peak_MB"]
    assert m_tp == m_sp * p["peak_ratio"]
    shapes_tp = {n: (s, h) for n, s, h, _ in tp_only}
    for region in p["tp_only_full_regions"]:
        assert list(shapes_tp[region]) == p["tp_only_full_shape"]
    assert all(stored for *_, stored in tp_only)
    shapes_sp = {n: (s, h) for n, s, h, _ in tp_sp}
    for region, shape in p["tp_sp_shapes"].items():
        assert list(shapes_sp[region]) == shape
    transient = [n for n, *_, stored in tp_sp if not stored]
    assert set(p["tp_sp_transient"]) <= set(transient)
    assert "row_linear" in transient and len(transient) == 4


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 64), st.integers(1, 64), st.sampled_from([1, 2, 4, 8, 16]), st.integers(1, 4))
def test_peak_ratio_is_t(sq, hq, t, b):
    s, h = sq * t, hq * t
    assert max_stored_bytes(shape_trace(s, h, t, False), b) == t * max_stored_bytes(shape_trace(s, h, t, True), b)


def test_worked_example_printed_values():
    g = load("lesson7_worked_example_70b.json")
    i, p = g["inputs"], g["printed"]
    s, b, h, t, L = i["s"], i["b"], i["h"], i["t"], i["layers"]
    tp = nontp_activation_bytes(s, b, h, t, sp=False)
    sp = nontp_activation_bytes(s, b, h, t, sp=True)
    assert tp == 10 * s * b * h == 1_342_177_280
    assert sp == 167_772_160
    assert round(float(tp) / 1e9, 2) == p["nontp_per_layer_GB"]
    assert round(float(L * tp) / 1e9, 1) == p["nontp_all_layers_GB"]
    assert s // t == p["sp_tokens_per_rank"]
    assert round(float(sp) / 1e6, 1) == p["sp_per_layer_MB"]
    assert round(float(L * sp) / 1e9, 1) == p["sp_all_layers_GB"]
    assert round(float(L * (tp - sp)) / 1e9) == p["saved_GB"]
    assert sp / tp == Fraction(*p["sp_fraction_of_tp_only"])


def test_trace_kept_tensors_hold_every_element_once():
    # Closed form independent of the table: the kept tensors of the TP-only
    # block are two full (s, h) token-wise tensors, two (s, h/t) TP tensors
    # and the all-reduced row output (s, h); with SP the token-wise tensors
    # shrink to s/t and the row output is no longer kept.  Boundary buffers
    # are never kept and exist only with SP.
    for s, h, t in ((4096, 4096, 8), (96, 40, 4), (7, 5, 1)):
        tp = shape_trace(s, h, t, sp=False)
        sp = shape_trace(s, h, t, sp=True)
        assert sum(sh * hh for _, sh, hh, k in tp if k) == 3 * s * h + 2 * s * (h // t)
        assert sum(sh * hh for _, sh, hh, k in sp if k) == 2 * (s // t) * h + 2 * s * (h // t)
        assert all(k for *_, k in tp) and len(tp) == 5
        assert sum(1 for *_, k in sp if not k) == 4 and len(sp) == 8


def test_comm_volume_closed_forms_and_saving():
    g = load("lesson7_comm_volume.json")
    s, b, h, t = 16384, 1, 8192, 8
    size = 2 * b * s * h
    v = comm_volume(t, size)
    assert v["block_tp"] == v["block_tp_sp"] == Fraction(4 * (t - 1), t) * size == 939_524_096
    assert v["all_reduce"] == v["reduce_scatter"] + v["all_gather"]
    assert (1 - Fraction(1, t)) * 100 == Fraction(g["printed"]["nontp_saving_at_t8_percent"]).limit_denominator()
    ops_tp, ops_sp = g["printed"]["ops_per_block_tp_only"], g["printed"]["ops_per_block_tp_sp"]
    assert v["block_tp"] == ops_tp["all_reduce"] * v["all_reduce"]
    assert v["block_tp_sp"] == ops_sp["all_gather"] * v["all_gather"] + ops_sp["reduce_scatter"] * v["reduce_scatter"]


def test_ring_simulation_volumes_and_allreduce_identity():
    # Integer-valued float64 data makes every sum exact regardless of order.
    rng = np.random.default_rng(0)
    for t in (2, 3, 4, 8):
        rows, h = 8 * t, 5
        xs = [rng.integers(-50, 50, (rows, h)).astype(np.float64) for _ in range(t)]
        size = xs[0].nbytes
        parts, sent_rs = ring_reduce_scatter(xs)
        total = sum(xs)
        for r in range(t):                      # g*: rank r keeps its summed slice
            assert np.array_equal(parts[r], np.array_split(total, t)[r])
        fulls, sent_ag = ring_all_gather(parts)
        for r in range(t):                      # all-reduce == all-gather(reduce-scatter)
            assert np.array_equal(fulls[r], total)
        v = comm_volume(t, size)
        assert all(sb == v["reduce_scatter"] for sb in sent_rs)
        assert all(sb == v["all_gather"] for sb in sent_ag)
        assert all(a + b == v["all_reduce"] for a, b in zip(sent_rs, sent_ag))
