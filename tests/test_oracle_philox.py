"""Pins of the oracle's Philox generator and of the dropout mask built on it.

* The round structure is fixed by numpy's Philox bit generator (a library
  implementation of Philox-4x64-10 from the same SC'11 paper): the same
  generic code at word width 64 must reproduce its stream.
* The Weyl key increments are closed forms (golden ratio, sqrt(3)).
* The vectorised 32-bit instance used by the region oracle must equal the
  generic one at width 32.
* The mask's statistics must match a Bernoulli(1-p) field: dropped fraction,
  independence of neighbouring channels and tokens, rank/seed sensitivity.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle.philox import PHILOX_CONSTANTS, philox4x32_10, philox_ref
from oracle.region import dropout_scale, dropout_threshold, keep_mask, token_index


@pytest.mark.parametrize("counter,key", [
    ([0, 0, 0, 0], [0, 0]),
    ([3, 4, 5, 6], [1, 2]),
    ([2 ** 64 - 2, 2 ** 64 - 1, 7, 2 ** 63], [0xDEADBEEFCAFEF00D, 0x0123456789ABCDEF]),
])
def test_width64_matches_numpy_philox(counter, key):
    bg = np.random.Philox(counter=np.array(counter, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = bg.random_raw(12)
    # numpy advances the 256-bit counter by one before producing each block of 4.
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    for blk in range(3):
        c = (c + 1) % (1 << 256)
        words = [(c >> (64 * i)) & (2 ** 64 - 1) for i in range(4)]
        assert list(philox_ref(words, key, width=64)) == [int(x) for x in raw[4 * blk:4 * blk + 4]]


def test_weyl_constants_closed_form():
    getcontext().prec = 60
    phi_frac = (Decimal(5).sqrt() - 1) / 2
    sqrt3_frac = Decimal(3).sqrt() - 1
    for w in (32, 64):
        assert PHILOX_CONSTANTS[w]["W0"] == int(phi_frac * (1 << w))
        assert PHILOX_CONSTANTS[w]["W1"] == int(sqrt3_frac * (1 << w))


def test_multipliers_are_odd_and_in_range():
    for w in (32, 64):
        for m in ("M0", "M1"):
            v = PHILOX_CONSTANTS[w][m]
            assert v & 1 and (1 << (w - 1)) < v < (1 << w)


def test_vectorised_equals_reference_width32():
    rng = np.random.default_rng(7)
    n = 300
    ctr = rng.integers(0, 2 ** 32, size=(n, 4), dtype=np.uint64)
    key = rng.integers(0, 2 ** 32, size=(n, 2), dtype=np.uint64)
    ctr[0] = 0
    key[0] = 0
    ctr[1] = 2 ** 32 - 1
    key[1] = 2 ** 32 - 1
    out = philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], key[:, 0], key[:, 1])
    for i in range(n):
        ref = philox_ref(ctr[i], key[i], width=32)
        assert tuple(int(o[i]) for o in out) == ref


def test_round_count_matters():
    # 10 rounds differ from 7 (catches a wrong round count in a stream that is
    # otherwise well mixed).
    assert philox_ref([1, 2, 3, 4], [5, 6], 32, 10) != philox_ref([1, 2, 3, 4], [5, 6], 32, 7)


def test_threshold_and_scale():
    assert dropout_threshold(0.0) == 0
    # p = 0.1 is taken as float32(0.1) = 0.100000001490116...
    assert dropout_threshold(0.1) == math.floor(float(np.float32(0.1)) * 2 ** 32) == 429496736
    assert dropout_threshold(0.5) == 2 ** 31
    assert dropout_scale(0.1) == np.float32(1 / (1 - float(np.float32(0.1))))
    assert dropout_scale(0.0) == np.float32(1.0)


def test_dropped_fraction_within_5_sigma():
    T, h, p = 2048, 8192, 0.1
    keep = keep_mask(0x5EED0002, p, token_index(T, 8, 0), h)
    n = keep.size
    dropped = n - int(keep.sum())
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(dropped - n * p) < 5 * sigma


def _pair_chi2(a: np.ndarray, b: np.ndarray, p: float) -> float:
    n = a.size
    obs = np.array([np.sum(a & b), np.sum(a & ~b), np.sum(~a & b), np.sum(~a & ~b)], dtype=np.float64)
    q = 1 - p
    exp = n * np.array([q * q, q * p, p * q, p * p])
    return float(np.sum((obs - exp) ** 2 / exp))


def test_neighbour_independence_chi2():
    # 3 degrees of freedom; chi2 > 30 has probability < 2e-6 for independent fields.
    T, h, p = 512, 4096, 0.1
    keep = keep_mask(12345, p, token_index(T, 8, 3), h)
    assert _pair_chi2(keep[:, :-1], keep[:, 1:], p) < 30      # channel j vs j+1
    assert _pair_chi2(keep[:, 3:-1:4], keep[:, 4::4], p) < 30  # across Philox blocks
    assert _pair_chi2(keep[:-1, :], keep[1:, :], p) < 30      # token i vs i+1


def test_mask_depends_on_seed_token_and_channel_only():
    h, p = 64, 0.5
    g = np.array([0, 1, 2 ** 32 + 1, 5], dtype=np.int64)
    m1 = keep_mask(99, p, g, h)
    m2 = keep_mask(99, p, g[::-1].copy(), h)[::-1]
    assert np.array_equal(m1, m2)                       # row order does not matter
    assert not np.array_equal(m1, keep_mask(100, p, g, h))
    assert not np.array_equal(m1[1], m1[2])             # hi32 of the token index is used
    assert not np.array_equal(keep_mask(1 << 32, p, g, h), keep_mask(0, p, g, h))  # hi32 of seed


def test_p_zero_keeps_everything():
    assert keep_mask(1, 0.0, np.arange(4), 16).all()
