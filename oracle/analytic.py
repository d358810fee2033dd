"""Analytic memory and communication model of Megatron TP+SP (test infrastructure only).

Source: hpc.payai.win lesson 7 "Sequence parallelism".
  * Code exercise (shape trace) and its answer: the activation shapes of one
    block's regions with and without SP, which tensors are kept for the
    backward and which are communication buffers, and the peak kept
    activation in bf16 (printed: 33.6 MB without SP, 4.2 MB with SP at
    s = h = 4096, t = 8).  Modelled below as a per-region sharding table plus
    separate boundary and stored-for-backward rules.
  * Section 4: ring all-reduce = reduce-scatter then all-gather; per rank
    V_AR = 2(t-1)/t * Size and V_RS = V_AG = (t-1)/t * Size; a block moves
    2 all-reduces without SP and 2 all-gathers + 2 reduce-scatters with SP,
    both 4(t-1)/t * (2bsh) bytes.
  * Worked example (70B model): the non-TP part of the per-layer stored
    activations is about 10sbh bytes, and SP divides it by t.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Tuple

import numpy as np

Tensor = Tuple[str, int, int, bool]   # (label, s, h, kept for the backward)

# The regions one block's forward passes through, in order (the lesson's code
# exercise traces these five).  Each region is described by which axis the
# tensor-parallel degree divides in its output, with sequence parallelism on
# and off.  Token-wise ops (LayerNorm, dropout) sit in the non-TP region:
# sequence parallelism gives every rank s/t of the tokens with all h channels
# (section 2 and section 3), and without it they hold the whole (s, h).  The
# column-parallel linear divides the hidden axis, the activation after it is
# element-wise, and the row-parallel linear's output has the full (s, h) again.
BLOCK = ("layernorm", "col_linear", "gelu", "row_linear", "dropout")
SPLIT_AXIS = {            # region: (axis divided by t with SP, axis divided by t without SP)
    "layernorm": ("s", None),
    "col_linear": ("h", "h"),
    "gelu": ("h", "h"),
    "row_linear": (None, None),
    "dropout": ("s", None),
}

# With SP the block crosses the SP/TP boundary twice (section 3.A): the
# all-gather g restores the whole sequence before the column-parallel
# linear, and after the row-parallel linear its full-h output is reduced and
# cut back to the rank's s/t tokens by the reduce-scatter g*.  Those tensors
# are communication or temporary buffers: (position, region, label, axis
# divided by t).
BOUNDARY = (
    ("before", "col_linear", "g_all_gather", None),
    ("after", "row_linear", "row_out", None),
    ("after", "row_linear", "g_star_reduce_scatter", "s"),
)


def _kept(region: str, sp: bool) -> bool:
    """Stored-for-backward rule: every region's output is kept, except the
    row-parallel linear's under SP, which is a partial sum that only lives
    until g* reduces it (its backward needs the region's input instead)."""
    return not (sp and region == "row_linear")


def _shape(axis, seq: int, hidden: int, tp: int) -> Tuple[int, int]:
    return (seq // tp, hidden) if axis == "s" else (seq, hidden // tp) if axis == "h" else (seq, hidden)


def shape_trace(seq: int, hidden: int, tp: int, sp: bool) -> List[Tensor]:
    """Activation tensors of one block's forward, in creation order:
    (label, s, h, kept).  Boundary buffers exist only with SP and are never kept."""
    out: List[Tensor] = []
    for region in BLOCK:
        if sp:
            out += [(lab, *_shape(ax, seq, hidden, tp), False)
                    for pos, reg, lab, ax in BOUNDARY if pos == "before" and reg == region]
        axis = SPLIT_AXIS[region][0 if sp else 1]
        out.append((region, *_shape(axis, seq, hidden, tp), _kept(region, sp)))
        if sp:
            out += [(lab, *_shape(ax, seq, hidden, tp), False)
                    for pos, reg, lab, ax in BOUNDARY if pos == "after" and reg == region]
    return out


def max_stored_bytes(trace: List[Tensor], batch: int = 1) -> int:
    """Peak kept activation: the largest kept tensor, at 2 bytes (bf16) per
    element of batch * s * h."""
    return max(2 * batch * s * h for _, s, h, kept in trace if kept)


def nontp_activation_bytes(s: int, b: int, h: int, t: int, sp: bool) -> Fraction:
    """The non-TP part of the per-layer stored activations of the 70B worked
    example: 10*s*b*h bytes (two LayerNorm inputs, the inputs of the QKV
    projection and of the first MLP linear, all bf16, and two one-byte
    dropout masks), divided by t under SP.  Returned exactly as a Fraction.
    (The worked example evaluates only this part of the per-layer formula;
    the formula's attention term needs the head count, which the example
    never gives, so it is not modelled here.)"""
    ln_inputs = 2 * (s * b * h) * 2          # two LayerNorm inputs, bf16
    gemm_inputs = 2 * (s * b * h) * 2        # QKV projection and MLP first-linear inputs
    dropout_masks = 2 * (s * b * h) * 1      # two dropout masks, one byte per element
    total = Fraction(ln_inputs + gemm_inputs + dropout_masks)
    return total / t if sp else total


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
