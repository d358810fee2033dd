"""Pins of the batch-planning oracle (oracle/batching.py): numpy's standard
deviation (a library routine) for the CV, hand-worked boundary cases, the
invariants that characterise the greedy buckets, and the link between the
padded shard layout and the region's ragged token index."""
import numpy as np
import pytest

import oracle.batching as B
import oracle.region as R


def check_cv_matches_numpy(B=B, seed=0, trials=400):
    """cv_within decides CV <= c exactly; away from the boundary it agrees
    with numpy's population std / mean."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(rng.integers(1, 40))
        x = rng.integers(0, 20000, n) if rng.random() < 0.5 else (4096 * rng.lognormal(0, 0.2, n)).astype(int)
        c_bp = int(rng.integers(0, 4000))
        cv = float(np.std(x) / np.mean(x)) if np.mean(x) > 0 else 0.0
        if abs(cv - c_bp / 1e4) < 1e-9:
            continue
        assert B.cv_within([int(v) for v in x], c_bp) == (cv <= c_bp / 1e4), (x, c_bp, cv)


def check_cv_hand_cases(B=B):
    """(1, 3): mean 2, population std 1, CV exactly 0.5 -> within 5000 bp, not
    within 4999; equal lengths have CV 0; an all-zero bucket counts as CV 0."""
    assert B.cv_within([1, 3], 5000) and not B.cv_within([1, 3], 4999)
    assert B.cv_within([7, 7, 7], 0) and B.cv_within([], 0) and B.cv_within([0, 0], 0)
    assert abs(B.length_cv([1, 3]) - 0.5) < 1e-15


def check_bucket_invariants(B=B, seed=1, trials=200):
    """The greedy buckets over the (length, index) order are exactly the
    partition into consecutive runs in which every prefix of a run is within
    the CV (and token budget) and no run can take the next sequence."""
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        n = int(rng.integers(0, 60))
        x = [int(v) for v in (rng.integers(1, 9000, n) if trial % 3 else 4096 * rng.lognormal(0, 0.5, n))]
        cv_bp = int(rng.choice([0, 500, 1500, 1800, 3000]))
        budget = int(rng.choice([0, 0, 20000, 60000]))
        order, starts = B.bucket_by_tokens(x, cv_bp, budget)
        assert sorted(order) == list(range(n))
        assert [(x[i], i) for i in order] == sorted((x[i], i) for i in range(n))
        assert starts[0] == 0 and starts[-1] == n and all(a < b for a, b in zip(starts, starts[1:])) or n == 0
        for k in range(len(starts) - 1):
            run = [x[i] for i in order[starts[k]:starts[k + 1]]]
            for m in range(2, len(run) + 1):
                assert B.cv_within(run[:m], cv_bp) and (budget == 0 or sum(run[:m]) <= budget)
            if k + 2 < len(starts):
                nxt = run + [x[order[starts[k + 1]]]]
                assert not (B.cv_within(nxt, cv_bp) and (budget == 0 or sum(nxt) <= budget))


def check_gate_thresholds(B=B):
    """The page's gate: SP unless the bucket's length CV exceeds 0.18 or the
    reduce-scatter wait share exceeds 0.22 (both bounds inclusive for SP)."""
    assert (B.GATE_CV_BP, B.GATE_RS_WAIT, B.MAX_CV_BP) == (1800, 0.22, 1500)
    at = [91, 109]              # mean 100, std 9: CV 0.09
    assert B.sp_gate(at, 0.22) and not B.sp_gate(at, 0.2200001)
    x = [82, 118]               # mean 100, std 18: CV exactly 0.18
    assert B.sp_gate(x, 0.0) and not B.sp_gate([81, 119], 0.0)


def check_layout_tiles_global_tokens(B=B, seed=2):
    """Padding to a multiple of t gives every rank the same T, and the
    region's ragged token index over all ranks enumerates exactly the padded
    global tokens."""
    rng = np.random.default_rng(seed)
    for t in (1, 2, 3, 8):
        x = [int(v) for v in rng.integers(0, 300, 9)]
        padded, cu, T = B.shard_layout(x, t)
        for a, p in zip(x, padded):
            assert p % t == 0 and a <= p < a + t
        assert cu[0] == 0 and T == cu[-1] == sum(padded) // t
        g = np.concatenate([R.token_index(T, t, r, np.array(cu)) for r in range(t)])
        assert np.array_equal(np.sort(g), np.arange(sum(padded)))


def test_cv_matches_numpy():
    check_cv_matches_numpy()


def test_cv_hand_cases():
    check_cv_hand_cases()


def test_bucket_invariants():
    check_bucket_invariants()


def test_gate_thresholds():
    check_gate_thresholds()


def test_layout_tiles_global_tokens():
    check_layout_tiles_global_tokens()


def test_bucket_example():
    order, starts = B.bucket_by_tokens([100, 4096, 4000, 110, 3900, 105, 8000])
    assert [[order[i] for i in range(a, b)] for a, b in zip(starts, starts[1:])] == [[0, 5, 3], [4, 2, 1], [6]]


# A planted mistake in each step must trip its pin.
from test_oracle_planted_mistakes import mutated  # noqa: E402

MUTATIONS = [
    ("sample_variance", "return 10 ** 8 * (n * s2 - s1 * s1) <= cv_bp * cv_bp * s1 * s1",
     "return 10 ** 8 * (n * s2 - s1 * s1) <= cv_bp * cv_bp * s1 * s1 * (n - 1) / max(n, 1) if n > 1 else True",
     check_cv_matches_numpy),
    ("strict_bound", "return 10 ** 8 * (n * s2 - s1 * s1) <= cv_bp * cv_bp * s1 * s1",
     "return 10 ** 8 * (n * s2 - s1 * s1) < cv_bp * cv_bp * s1 * s1", check_cv_hand_cases),
    ("descending", "order = sorted(range(len(lengths)), key=lambda i: (lengths[i], i))",
     "order = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))", check_bucket_invariants),
    ("budget_ignored", "fits = cv_within(cand, max_cv_bp) and (max_tokens == 0 or sum(cand) <= max_tokens)",
     "fits = cv_within(cand, max_cv_bp)", check_bucket_invariants),
    ("gate_ignores_wait", "return cv_within(lengths, max_cv_bp) and not (rs_wait_share > max_rs_wait_share)",
     "return cv_within(lengths, max_cv_bp)", check_gate_thresholds),
    ("no_padding", "padded = [-(-int(x) // t) * t for x in lengths]", "padded = [int(x) for x in lengths]",
     check_layout_tiles_global_tokens),
]


@pytest.mark.parametrize("name,find,replace,check", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_batching_mistake_is_caught(name, find, replace, check):
    Bm = mutated("oracle.batching", find, replace)
    with pytest.raises(AssertionError):
        check(B=Bm)
