"""Pins of the fp8 (e4m3) emulation in the oracle (CPU)."""
import numpy as np
import pytest
import torch

from oracle import fp8


def _torch_e4m3(x):
    t = torch.from_numpy(np.asarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_round_e4m3_matches_torch_float8_e4m3fn():
    g = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(fp8.round_e4m3(x), _torch_e4m3(x))


def test_round_e4m3_closed_forms():
    # largest finite, smallest subnormal, ties to even, saturation
    assert fp8.round_e4m3(448.0) == 448.0 and fp8.round_e4m3(1000.0) == 448.0
    assert fp8.round_e4m3(-1e9) == -448.0
    assert fp8.round_e4m3(2.0 ** -9) == 2.0 ** -9
    assert fp8.round_e4m3(2.0 ** -10) == 0.0          # tie between 0 and 2^-9 -> even (0)
    assert fp8.round_e4m3(3 * 2.0 ** -10) == 2.0 ** -8  # tie 1 vs 2 (x 2^-9) -> even (2)
    assert fp8.round_e4m3(1.0625) == 1.0              # 1 + 1/16 is halfway 1 .. 1.125 -> even
    assert fp8.round_e4m3(1.1875) == 1.25             # halfway 1.125 .. 1.25 -> even mantissa
    assert fp8.round_e4m3(17.0) == 16.0 and fp8.round_e4m3(19.0) == 20.0
    # every e4m3 value is a fixed point
    vals = [m * 2.0 ** -9 for m in range(8)] + [(1 + m / 8) * 2.0 ** e for e in range(-6, 9) for m in range(8)]
    vals = [v for v in vals if v <= 448]
    assert np.array_equal(fp8.round_e4m3(vals), vals)


def test_quantise_per_head_scale_and_range():
    g = np.random.Generator(np.random.PCG64(6))
    x = g.standard_normal((2, 50, 3, 8)).astype(np.float32)
    x[1, 7, 2, 3] = 40.0
    dq, s = fp8.quantise(x)
    assert s.shape == (2, 3) and s.dtype == np.float32
    assert s[1, 2] == np.float32(40.0) / np.float32(448.0)
    # the absmax element maps to the code 448 exactly
    assert dq[1, 7, 2, 3] == pytest.approx(40.0, rel=1e-7)
    # relative error of a 3-bit mantissa is at most 2^-4 for normal codes
    big = np.abs(x) > 0.05 * np.abs(x).max(axis=(1, 3), keepdims=True)
    rel = np.abs(dq - x) / np.abs(x)
    assert np.all(rel[big] <= 2.0 ** -4 + 1e-6)
