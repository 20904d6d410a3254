"""Pins for the oracle's number formats, against things other than itself:
PyTorch's CPU bfloat16 conversion (a library routine) and a float64 search
for the nearest bf16 neighbour."""
import numpy as np
import torch

from oracle import numerics


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _special_values():
    vals = [0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38,
            3.4028235e38, 1e-40, -1e-40, 1.4e-45, np.inf, -np.inf,
            65504.0, 1.0 + 2 ** -8 + 2 ** -23, 1.0 - 2 ** -24]
    bits = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x7F7FFFFF, 0x7F7F8000,
                     0x00008000, 0x00018000, 0x807F8000], dtype=np.uint32)
    return np.concatenate([np.array(vals, dtype=np.float32), bits.view(np.float32)])


def test_rne_matches_torch_on_random_and_special_values():
    g = np.random.default_rng(123)
    raw = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = np.concatenate([x[np.isfinite(x)], _special_values()])
    assert np.array_equal(numerics.f32_to_bf16(x), _torch_bf16_bits(x))


def test_rne_is_the_nearest_neighbour_ties_to_even():
    g = np.random.default_rng(7)
    raw = g.integers(0, 2 ** 32, size=20_000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties
    raw[:5000] = (raw[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = raw.view(np.float32)
    keep = np.isfinite(x) & (np.abs(x) < np.float32(3.3e38))
    x = x[keep]
    got = numerics.f32_to_bf16(x)
    for xi, gi in zip(x[:20000], got[:20000]):
        b = int(np.array([xi], dtype=np.float32).view(np.uint32)[0])
        lo = b >> 16                      # truncated magnitude
        hi = lo + 1                       # next magnitude up
        f = float(xi)
        vlo = float(np.array([lo << 16], dtype=np.uint32).view(np.float32)[0])
        vhi = float(np.array([(hi << 16) & 0xFFFFFFFF], dtype=np.uint32).view(np.float32)[0])
        dlo, dhi = abs(f - vlo), abs(vhi - f)
        if dlo < dhi:
            want = lo
        elif dhi < dlo:
            want = hi
        else:
            want = lo if lo % 2 == 0 else hi
        assert int(gi) == want, (f, hex(b))


def test_nan_stays_nan_and_inf_is_kept():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf], dtype=np.float32)
    y = numerics.bf16_to_f32(numerics.f32_to_bf16(x))
    assert np.isnan(y[0]) and np.isnan(y[1])
    assert y[2] == np.inf and y[3] == -np.inf


def test_bf16_widening_is_exact_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = numerics.bf16_to_f32(bits)
    finite = np.isfinite(f)
    # widening then narrowing returns the same pattern (widening is exact)
    assert np.array_equal(numerics.f32_to_bf16(f[finite]), bits[finite])
    # and agrees with PyTorch's own widening
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(t[finite].view(np.uint32), f[finite].view(np.uint32))


def test_round_to_nearest_examples():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: the even neighbour is 1
    assert numerics.f32_to_bf16(np.float32([1.00390625]))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert numerics.f32_to_bf16(np.float32([1.01171875]))[0] == 0x3F82
    # just above the tie rounds up
    assert numerics.f32_to_bf16(np.array([0x3F808001], dtype=np.uint32).view(np.float32))[0] == 0x3F81
    # the largest finite fp32 rounds to infinity in bf16
    assert numerics.f32_to_bf16(np.array([0x7F7FFFFF], dtype=np.uint32).view(np.float32))[0] == 0x7F80


def test_u8_widening():
    v = np.arange(256, dtype=np.uint8)
    assert np.array_equal(numerics.u8_to_f32(v), np.arange(256, dtype=np.float32))
