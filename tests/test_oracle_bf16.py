"""Pins of the oracle's bf16 codec against torch's CPU float32 -> bfloat16 cast
(a library implementation of IEEE round-to-nearest-even) and exact decoding."""
import numpy as np
import pytest
import torch

from oracle.bf16 import bf16_to_f32, bf16_ulp, f32_to_bf16


def torch_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_random_values_match_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-40, 40, 200_000))).astype(np.float32)
    assert np.array_equal(f32_to_bf16(x), torch_bits(x))


def test_every_tie_and_neighbour_pattern():
    # All 2^16 values of the dropped half over a few kept patterns (even/odd last
    # kept bit, both signs, the top finite binade and the subnormals).
    low = np.arange(1 << 16, dtype=np.uint32)
    for hi in (0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x7F7E, 0x7F7F, 0x0000, 0x0001, 0x8000, 0x007F):
        u = (np.uint32(hi) << np.uint32(16)) | low
        x = u.view(np.float32)
        assert np.array_equal(f32_to_bf16(x), torch_bits(x)), hex(hi)


def test_ties_go_to_even_by_hand():
    # 1 + 2^-8 lies halfway between bf16 1.0 (even) and 1 + 2^-7 (odd): rounds down.
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): rounds up.
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert list(f32_to_bf16(x)) == [0x3F80, 0x3F82, 0xBF80]


def test_overflow_to_inf_and_nan():
    big = np.array([3.4e38, -3.4e38, np.inf, -np.inf, np.nan], dtype=np.float32)
    out = f32_to_bf16(big)
    assert out[0] == 0x7F80 and out[1] == 0xFF80 and out[2] == 0x7F80 and out[3] == 0xFF80
    assert np.isnan(bf16_to_f32(out[4:]))[0]


def test_decode_is_exact_and_roundtrips():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f32(bits)
    finite = np.isfinite(vals)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(vals[finite], ref[finite])
    assert np.array_equal(f32_to_bf16(vals[finite]), bits[finite])


@pytest.mark.parametrize("x,ulp", [(1.0, 2 ** -7), (1.99, 2 ** -7), (2.0, 2 ** -6), (7.9, 2 ** -5), (8.0, 2 ** -4), (-0.3, 2 ** -9)])
def test_ulp(x, ulp):
    assert bf16_ulp(np.array([x]))[0] == ulp
