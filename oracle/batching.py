"""CPU oracle of the host-side batch planning around the SP region (test
infrastructure only): length buckets, the SP gate and the packed shard
layout.

Source: coreui.cn, "Why Sequence Parallel saves memory but makes throughput
jitter: from reduce-scatter to the LayerNorm boundary", section "stabilise
the shapes first, then define the LayerNorm shard contract".  Its step
function first groups the batch into length buckets whose length
coefficient of variation is at most 0.15 (bucket_by_tokens with
max_cv=0.15), then falls back to tensor parallelism alone when a bucket's
length CV exceeds 0.18 or the measured reduce-scatter wait share exceeds
0.22; figure 3's table credits the buckets with 0.91x -> 0.97x throughput.

Readings where the page is silent (each listed in the design notes):
  * length CV = population standard deviation / mean of the sequence
    lengths in a bucket (0 for an empty or all-zero bucket);
  * a bucket is a run of the batch sorted by (length, original index),
    grown greedily: the next sequence joins while the run's CV stays
    <= max_cv and, when a token budget is given, the run's token total stays
    within it; otherwise it starts the next bucket;
  * CV thresholds are given in basis points (1500 = 0.15) and the test
    "CV <= c" is decided exactly in integers:
        n * sum(x^2) - sum(x)^2 <= (c_bp / 10^4)^2 * sum(x)^2
    (population variance times n^2 against c^2 * mean^2 times n^2);
  * the SP split gives rank r the r-th of t equal slices of every sequence,
    so each sequence is padded up to a multiple of t and every rank holds
    the same number of tokens, sum(padded) / t.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

MAX_CV_BP = 1500          # bucket_by_tokens(max_cv=0.15)
GATE_CV_BP = 1800         # fall back to TP alone above a length CV of 0.18
GATE_RS_WAIT = 0.22       # ... or above a reduce-scatter wait share of 0.22


def length_cv(lengths: Sequence[int]) -> float:
    """Population std / mean (reporting only; decisions use cv_within)."""
    n = len(lengths)
    if n == 0:
        return 0.0
    s1 = sum(lengths)
    if s1 == 0:
        return 0.0
    mean = s1 / n
    var = sum((x - mean) ** 2 for x in lengths) / n
    return var ** 0.5 / mean


def cv_within(lengths: Sequence[int], cv_bp: int) -> bool:
    """CV(lengths) <= cv_bp / 10^4, decided exactly (Python integers)."""
    n = len(lengths)
    s1 = sum(int(x) for x in lengths)
    s2 = sum(int(x) * int(x) for x in lengths)
    return 10 ** 8 * (n * s2 - s1 * s1) <= cv_bp * cv_bp * s1 * s1


def bucket_by_tokens(lengths: Sequence[int], max_cv_bp: int = MAX_CV_BP,
                     max_tokens: int = 0) -> Tuple[List[int], List[int]]:
    """Greedy buckets over the batch sorted by (length, index).

    Returns (order, starts): order lists the original indices bucket by
    bucket, and bucket k is order[starts[k]:starts[k+1]].  max_tokens = 0
    means no token budget; a single sequence above the budget still forms a
    bucket of its own."""
    order = sorted(range(len(lengths)), key=lambda i: (lengths[i], i))
    starts: List[int] = []
    cur: List[int] = []
    for pos, i in enumerate(order):
        cand = [lengths[j] for j in cur] + [lengths[i]]
        fits = cv_within(cand, max_cv_bp) and (max_tokens == 0 or sum(cand) <= max_tokens)
        if cur and not fits:
            cur = []
        if not cur:
            starts.append(pos)
        cur.append(i)
    starts.append(len(order))
    return order, starts


def sp_gate(lengths: Sequence[int], rs_wait_share: float, max_cv_bp: int = GATE_CV_BP,
            max_rs_wait_share: float = GATE_RS_WAIT) -> bool:
    """True: run the bucket with sequence parallelism; False: fall back to
    tensor parallelism alone (length CV above the gate, or too much
    reduce-scatter wait)."""
    return cv_within(lengths, max_cv_bp) and not (rs_wait_share > max_rs_wait_share)


def shard_layout(lengths: Sequence[int], t: int) -> Tuple[List[int], List[int], int]:
    """Pad every sequence to a multiple of t; return (padded lengths, local
    cu_seqlens of one rank, local token count T = sum(padded) / t)."""
    padded = [-(-int(x) // t) * t for x in lengths]
    cu = [0]
    for x in padded:
        cu.append(cu[-1] + x // t)
    return padded, cu, cu[-1]
