"""bfloat16 storage codec of the oracle (test infrastructure only).

bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of an
IEEE-754 binary32 value, so every bf16 value is the binary32 value whose low 16
bits are zero.  Decoding is therefore exact.  Encoding rounds to nearest with
ties to even (the IEEE-754 default rounding attribute).

The encoder below is that definition written out: the two bf16 neighbours of
a finite binary32 ``x`` are ``x`` with its low 16 bits cleared (towards zero)
and the next bf16 away from zero; it picks the nearer one, and on an exact tie
the one whose last kept bit is 0.  Stepping past the largest finite bf16 lands
on infinity, as IEEE rounding requires.  NaN inputs map to a quiet NaN with the
input's sign.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values -> uint16 bf16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    toward_zero = u >> np.uint32(16)                  # bf16 with the low bits dropped
    away = toward_zero + np.uint32(1)                 # next bf16 away from zero
    rest = u & np.uint32(0xFFFF)                      # dropped part, in units of 2^-16 ulp
    half = np.uint32(0x8000)
    pick_away = (rest > half) | ((rest == half) & ((toward_zero & np.uint32(1)) == 1))
    out = np.where(pick_away, away, toward_zero).astype(np.uint32)
    is_nan = np.isnan(x)
    if is_nan.any():
        out = np.where(is_nan, (u >> np.uint32(16)) | np.uint32(0x0040), out)
    return out.astype(np.uint16)


def round_f32_to_bf16_value(x: np.ndarray) -> np.ndarray:
    """float32 -> the float32 value of its bf16 rounding."""
    return bf16_to_f32(f32_to_bf16(x))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (float64): 2^(e-7) for |x| in [2^e, 2^(e+1)),
    with the subnormal spacing 2^-133 as the floor."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))
