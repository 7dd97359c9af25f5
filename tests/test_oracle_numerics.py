"""Pins for the oracle's storage rounding (CPU only).

round_fmt is checked against independent conversions (numpy's float16 and
float32 casts, torch's float32 -> bfloat16 cast) and hand-computed IEEE cases.
"""
import numpy as np
import pytest
import torch

from oracle import round_fmt


def _samples(n=200_000, seed=0):
    g = np.random.default_rng(seed)
    mag = 10.0 ** g.uniform(-12, 6, size=n)
    sgn = np.where(g.random(n) < 0.5, -1.0, 1.0)
    return sgn * mag


@pytest.mark.parametrize("fmt,npdt", [("f16", np.float16), ("f32", np.float32)])
def test_round_matches_numpy_cast(fmt, npdt):
    x = _samples()
    with np.errstate(over="ignore"):
        ref = x.astype(npdt).astype(np.float64)
    np.testing.assert_array_equal(round_fmt(x, fmt), ref)


def test_round_f16_ties_and_edges():
    cases = {
        1.0 + 2.0 ** -11: 1.0,                      # tie -> even mantissa
        1.0 + 3 * 2.0 ** -11: 1.0 + 2.0 ** -9,      # tie -> even (up)
        65519.0: 65504.0,
        65520.0: np.inf,                            # exactly half an ulp above max -> inf
        -65520.0: -np.inf,
        2.0 ** -25: 0.0,                            # half the smallest subnormal, tie to 0
        3 * 2.0 ** -26: 2.0 ** -24,
        2.0 ** -24: 2.0 ** -24,
    }
    x = np.array(list(cases.keys()))
    np.testing.assert_array_equal(round_fmt(x, "f16"), np.array(list(cases.values())))


def test_round_bf16_matches_torch_on_f32_inputs():
    g = np.random.default_rng(1)
    x = _samples(seed=2).astype(np.float32)
    # add exact ties: values halfway between two bf16 neighbours
    base = g.integers(0x3F80, 0x4780, size=2000).astype(np.uint32) << 16
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_fmt(x.astype(np.float64), "bf16"), ref)


def test_round_bf16_edges():
    big = 2.0 ** 127 * (2 - 2.0 ** -7)              # largest finite bf16
    cases = {
        1.0 + 2.0 ** -8: 1.0,
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,
        big: big,
        2.0 ** 127 * (2 - 2.0 ** -8): np.inf,       # max + half ulp -> inf (ties to even)
        2.0 ** -133: 2.0 ** -133,                   # smallest bf16 subnormal
        2.0 ** -134: 0.0,
    }
    x = np.array(list(cases.keys()))
    np.testing.assert_array_equal(round_fmt(x, "bf16"), np.array(list(cases.values())))


def test_round_passes_nonfinite_and_identity():
    x = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0])
    for fmt in ("f16", "bf16", "f32"):
        r = round_fmt(x, fmt)
        assert np.isnan(r[0]) and r[1] == np.inf and r[2] == -np.inf and r[3] == 0.0
    y = _samples(100)
    np.testing.assert_array_equal(round_fmt(y, "f64"), y)
