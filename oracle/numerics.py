"""Number formats for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32 word: 1 sign, 8 exponent and 7
fraction bits.  Widening bf16 -> fp32 is exact (append 16 zero bits).
Narrowing fp32 -> bf16 rounds to nearest, ties to the even neighbour,
written out from that definition on the 16 discarded bits; a NaN stays a
NaN (its quiet bit is set).  u8 values widen to the float of the same
integer.

Pinned in tests/test_oracle_numerics.py against PyTorch's CPU bf16
conversion and against a float64 nearest-neighbour search.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    upper = (bits >> np.uint32(16)).astype(np.uint32)       # truncated toward zero
    lower = bits & np.uint32(0xFFFF)                        # the discarded half
    half = np.uint32(0x8000)
    odd = (upper & np.uint32(1)) == 1
    up = (lower > half) | ((lower == half) & odd)
    # Incrementing the magnitude carries into the exponent (and to infinity)
    # exactly as rounding up to the next representable magnitude should.
    out = upper + up.astype(np.uint32)
    nan = np.isnan(x)
    out = np.where(nan, upper | np.uint32(0x0040), out)
    return out.astype(np.uint16)


def u8_to_f32(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.uint8).astype(np.float32)


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f32(arr)
    if dtype == "u8":
        return u8_to_f32(arr)
    raise ValueError(dtype)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16(x)
    raise ValueError(f"no stores of dtype {dtype}")


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """The fp32 value a store of dtype followed by a reload gives back."""
    return decode(encode(x, dtype), dtype)
