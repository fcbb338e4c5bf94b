"""Pins for the oracle's storage rounding.

bfloat16: checked against torch's float32 -> bfloat16 conversion (a library
routine, round to nearest even) on float32-exact inputs, plus hand-derived
float64 tie cases that a float32 detour would get wrong.
"""
import numpy as np
import pytest
import torch

from oracle.rounding import round_bf16, to_storage


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_matches_torch_on_float32_inputs():
    g = np.random.default_rng(0)
    x = np.clip(g.standard_normal(200_000) * np.exp(g.uniform(-90, 88, 200_000)), -3e38, 3e38).astype(np.float32)
    # exact halfway cases between neighbouring bfloat16 values
    bits = g.integers(0, 2**32, 50_000, dtype=np.uint64).astype(np.uint32)
    bits = (bits & 0xFFFF0000) | 0x8000
    ties = bits.view(np.float32)
    ties = ties[np.isfinite(ties)]
    sub = (g.standard_normal(10_000) * 1e-39).astype(np.float32)   # float32 subnormals
    for arr in (x, ties, sub):
        np.testing.assert_array_equal(round_bf16(arr.astype(np.float64)), _torch_bf16(arr))


def test_bf16_float64_ties_and_specials():
    one = 1.0
    assert round_bf16([one + 2.0**-8])[0] == 1.0                     # tie -> even (1.0)
    assert round_bf16([one + 3 * 2.0**-8])[0] == 1.0 + 2.0**-6       # tie -> even (up)
    assert round_bf16([one + 2.0**-8 + 2.0**-40])[0] == 1.0 + 2.0**-7  # just above the tie
    assert round_bf16([-(one + 2.0**-8 + 2.0**-40)])[0] == -(1.0 + 2.0**-7)
    big = (2.0 - 2.0**-8) * 2.0**127                                   # halfway past the max
    assert np.isinf(round_bf16([big])[0]) and round_bf16([big])[0] > 0
    assert round_bf16([np.nextafter(big, 0)])[0] == (2.0 - 2.0**-7) * 2.0**127
    r = round_bf16([np.nan, np.inf, -np.inf, 0.0, -0.0])
    assert np.isnan(r[0]) and r[1] == np.inf and r[2] == -np.inf
    assert r[3] == 0.0 and np.signbit(r[4])


def test_f32_and_f64_storage():
    x = np.array([1.0 + 2.0**-30, np.pi, -1e-50])
    np.testing.assert_array_equal(to_storage(x, "f32"), x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(to_storage(x, "f64"), x)
    with pytest.raises(ValueError):
        to_storage(x, "fp8")
