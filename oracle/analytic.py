"""Analytic memory and communication model of Megatron TP+SP (test infrastructure only).

Source: hpc.payai.win lesson 7 "Sequence parallelism".
  * Code exercise and its answer: a block is traced through the regions
    layernorm -> col_linear -> gelu -> row_linear -> dropout, tracking the
    activation shape (s, h).  Without SP every region sees the full sequence;
    the column-parallel linear splits h by tp, the row-parallel linear restores
    it.  With SP the layernorm and dropout regions hold s/tp tokens; an
    all-gather (g) restores the full sequence before the column-parallel linear
    and a reduce-scatter (g*) cuts the row-parallel output back to s/tp.  The
    g / row-output / g* buffers are transient; every region's own activation is
    stored for the backward.  The peak stored activation in bf16 is
    max(b*s*h*2) over stored entries.
  * Section 4: ring all-reduce = reduce-scatter then all-gather; per rank
    V_AR = 2(t-1)/t * Size and V_RS = V_AG = (t-1)/t * Size; a block moves
    2 all-reduces without SP and 2 all-gathers + 2 reduce-scatters with SP,
    both 4(t-1)/t * (2bsh) bytes.
  * Worked example: per-layer activations sbh(10 + 24/t + 5as/(ht)) bytes,
    whose non-TP part is about 10sbh (two LayerNorm inputs 4sbh, the inputs of
    the QKV projection and the first MLP linear 4sbh, two 1-byte dropout masks
    2sbh); SP divides that part by t.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Tuple

import numpy as np

TraceEntry = Tuple[str, int, int, bool]   # (region, s, h, stored_for_backward)

REGIONS = ("layernorm", "col_linear", "gelu", "row_linear", "dropout")


def trace_block(seq: int, hidden: int, tp: int, enable_sp: bool) -> List[TraceEntry]:
    """Activation shapes of one block's forward, in region order."""
    out: List[TraceEntry] = []
    s_full, h_full = seq, hidden
    s_sp = seq // tp if enable_sp else seq          # sequence length inside the SP region
    for region in REGIONS:
        if region == "layernorm":
            out.append((region, s_sp, h_full, True))
        elif region == "col_linear":
            if enable_sp:                             # g: all-gather along s into the TP region
                out.append(("g_all_gather", s_full, h_full, False))
            out.append((region, s_full, h_full // tp, True))
        elif region == "gelu":
            out.append((region, s_full, h_full // tp, True))
        elif region == "row_linear":
            # Without SP the all-reduced row output is the next region's stored input.
            # With SP it is a partial sum, transient until g* reduces and splits it.
            out.append((region, s_full, h_full, not enable_sp))
            if enable_sp:
                out.append(("row_out", s_full, h_full, False))
                out.append(("g_star_reduce_scatter", s_sp, h_full, False))
        elif region == "dropout":
            out.append((region, s_sp, h_full, True))
    return out


def bf16_bytes(s: int, h: int, batch: int = 1) -> int:
    return batch * s * h * 2


def max_stored_bytes(trace: List[TraceEntry], batch: int = 1) -> int:
    """Peak stored (kept for backward) activation in bf16 bytes."""
    return max(bf16_bytes(s, h, batch) for _, s, h, stored in trace if stored)


def nontp_activation_bytes(s: int, b: int, h: int, t: int, sp: bool) -> Fraction:
    """The non-TP part of the per-layer stored activations: 10*s*b*h bytes,
    divided by t under SP.  Returned exactly as a Fraction."""
    ln_inputs = 2 * (s * b * h) * 2          # two LayerNorm inputs, bf16
    gemm_inputs = 2 * (s * b * h) * 2        # QKV projection and MLP first-linear inputs
    dropout_masks = 2 * (s * b * h) * 1      # two dropout masks, one byte per element
    total = Fraction(ln_inputs + gemm_inputs + dropout_masks)
    return total / t if sp else total


def activation_bytes_per_layer(s: int, b: int, h: int, t: int, a: int, sp: bool) -> Fraction:
    """sbh(10 + 24/t + 5as/(ht)) without SP; the 10sbh term divided by t with SP.
    Exact (Fraction).  The head count a is a free parameter."""
    sbh = Fraction(s * b * h)
    tp_part = sbh * (Fraction(24, t) + Fraction(5 * a * s, h * t))
    return nontp_activation_bytes(s, b, h, t, sp) + tp_part


def comm_volume(t: int, size: int) -> dict:
    """Per-rank bytes of the ring collectives and of one block's forward."""
    rs = Fraction(t - 1, t) * size
    ag = Fraction(t - 1, t) * size
    ar = 2 * Fraction(t - 1, t) * size
    return dict(all_reduce=ar, reduce_scatter=rs, all_gather=ag,
                block_tp=2 * ar, block_tp_sp=2 * (ag + rs))


def ring_reduce_scatter(xs: List[np.ndarray]):
    """Simulated ring reduce-scatter over len(xs) ranks.  Each rank's array is
    split into t equal chunks along axis 0; in each of t-1 steps every rank
    sends one partially reduced chunk to its right neighbour, which adds its
    own copy.  Returns (chunks, bytes_sent_per_rank): rank r ends with the full
    sum of chunk r."""
    t = len(xs)
    chunks = [np.array_split(x.copy(), t) for x in xs]
    sent = [0] * t
    for step in range(t - 1):
        msgs = []
        for r in range(t):
            c = (r - step - 1) % t                 # chunk rank r forwards this step
            msgs.append((c, chunks[r][c].copy()))
            sent[r] += chunks[r][c].nbytes
        for r in range(t):
            c, data = msgs[(r - 1) % t]            # receive from the left neighbour
            chunks[r][c] = chunks[r][c] + data
    return [chunks[r][r] for r in range(t)], sent


def ring_all_gather(parts: List[np.ndarray]):
    """Simulated ring all-gather: rank r starts with chunk r; in t-1 steps each
    rank forwards the chunk it received last.  Returns (full arrays, bytes_sent_per_rank)."""
    t = len(parts)
    have = [{r: parts[r].copy()} for r in range(t)]
    sent = [0] * t
    for step in range(t - 1):
        msgs = []
        for r in range(t):
            c = (r - step) % t
            msgs.append((c, have[r][c]))
            sent[r] += have[r][c].nbytes
        for r in range(t):
            c, data = msgs[(r - 1) % t]
            have[r][c] = data.copy()
    return [np.concatenate([have[r][c] for c in range(t)]) for r in range(t)], sent
