"""Counter-based random numbers for the synthetic workloads.

Every value is a pure function of (seed, stream, index), so any slice of a
tensor can be regenerated without generating what precedes it, and the result
never depends on NumPy's distribution code.

The mixing function is splitmix64's output stage (Steele, Lea and Flood,
"Fast Splittable Pseudorandom Number Generators", OOPSLA 2014): add a
Weyl-sequence increment, then xor-shift-multiply three times.  Uniforms take
the top 53 bits; normals use the Box-Muller transform (cosine branch only).

This module holds input generation only.  It contains none of the arithmetic
of the fused groups or of the buckets.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = _mix(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]
        t = _mix(np.array([(stream * 0x632BE59BD9B4E019 + 1) & 0xFFFFFFFFFFFFFFFF],
                          dtype=np.uint64))[0]
        return np.uint64(s ^ t)


def bits64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit words for counters start .. start+count-1."""
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = _key(seed, stream) + (idx + np.uint64(1)) * _GOLDEN
    return _mix(z)


def uniform(seed: int, stream: int, count: int, lo: float = 0.0, hi: float = 1.0,
            start: int = 0) -> np.ndarray:
    """float64 draws from the half-open interval [lo, hi)."""
    u = (bits64(seed, stream, start, count) >> np.uint64(11)).astype(np.float64)
    u *= 2.0 ** -53
    return lo + (hi - lo) * u


def normal(seed: int, stream: int, count: int, mean: float = 0.0, std: float = 1.0,
           start: int = 0) -> np.ndarray:
    """float64 normal draws; element i uses counters 2(start+i) and 2(start+i)+1."""
    w = bits64(seed, stream, 2 * start, 2 * count)
    u = (w >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    u1 = 1.0 - u[0::2]          # (0, 1]: log is finite
    u2 = u[1::2]
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return mean + std * z
