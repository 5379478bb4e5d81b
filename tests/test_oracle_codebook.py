"""Pins of the oracle's Gaussian Lloyd-Max codebooks (CPU only)."""

import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")


def _golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            rows[(int(line[0]), line[1])] = [float(x) for x in line[2:]]
    return rows


def test_one_bit_closed_form():
    t, c, mse = codebook.solve(1)
    assert t.tolist() == [0.0]
    assert c[1] == pytest.approx(math.sqrt(2.0 / math.pi), rel=1e-15)
    assert c[0] == -c[1]
    assert mse == pytest.approx(1.0 - 2.0 / math.pi, rel=1e-13)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_textbook_table(bits):
    rows = _golden()
    t, c, mse = codebook.solve(bits)
    half = 1 << (bits - 1)
    np.testing.assert_allclose(t[half:], rows[(bits, "thr")], rtol=0, atol=6e-4 if bits < 4 else 2e-3)
    np.testing.assert_allclose(c[half:], rows[(bits, "out")], rtol=0, atol=6e-4 if bits < 4 else 2e-3)
    assert mse == pytest.approx(rows[(bits, "mse")][0], abs=2e-5 if bits < 4 else 1e-5)


@pytest.mark.parametrize("bits", range(1, 9))
def test_fixed_point_by_quadrature(bits):
    """Centroids are conditional means and thresholds midpoints, checked by numerical integration."""
    t, c, mse = codebook.solve(bits)
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-12)
    phi = stats.norm.pdf
    half = len(c) // 2
    total = 0.0
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        lo, hi = max(a, -12.0), min(b, 12.0)
        mass = integrate.quad(phi, lo, hi, epsabs=0, epsrel=1e-13)[0]
        mean = integrate.quad(lambda x: x * phi(x), lo, hi, epsabs=0, epsrel=1e-13)[0] / mass
        if k >= half:
            assert c[k] == pytest.approx(mean, rel=1e-9, abs=1e-12)
        total += integrate.quad(lambda x: (x - c[k]) ** 2 * phi(x), lo, hi, epsabs=0, epsrel=1e-12)[0]
    assert mse == pytest.approx(total, rel=1e-8)


def test_high_rate_asymptote():
    """Panter-Dite: D(b) -> (pi*sqrt(3)/2) * 4^-b for the unit Gaussian."""
    pd = math.pi * math.sqrt(3.0) / 2.0
    ratios = [codebook.solve(b)[2] * 4.0 ** b / pd for b in (5, 6, 7, 8)]
    assert all(r < 1.0 for r in ratios) and np.all(np.diff(ratios) > 0)
    assert ratios[-1] == pytest.approx(1.0, abs=0.01)


def test_tables_symmetric_monotone_convex():
    d32 = codebook.distortion32()
    assert d32[0] == 1.0
    gains = d32[:-1] - d32[1:]
    assert np.all(np.diff(gains) < 0), "D(b) - D(b+1) must strictly decrease (convexity)"
    for b in range(1, 9):
        t32, c32 = codebook.thresholds32(b), codebook.centroids32(b)
        assert t32.dtype == np.float32 and c32.dtype == np.float32
        assert np.all(np.diff(t32) > 0) and np.all(np.diff(c32) > 0)
        np.testing.assert_array_equal(t32, -t32[::-1])
        np.testing.assert_array_equal(c32, -c32[::-1])
        assert np.all(c32[:-1] < t32) and np.all(t32 < c32[1:])


@pytest.mark.parametrize("bits", range(1, 9))
def test_fp16_reconstruction_levels(bits):
    """fp16 levels are the nearest-even fp16 of the fp32 centroids; moving off the optimal levels can
    only raise the MSE, by under 1e-4 relative up to 5 bits and under 2% at 8 bits."""
    c32 = codebook.centroids32(bits).astype(np.float64)
    c16 = codebook.levels16(bits)
    assert np.all(np.abs(c16 - c32) <= 2.0 ** -11 * np.abs(c32))
    np.testing.assert_array_equal(c16, -c16[::-1])
    t, _, mse = codebook.solve(bits)
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    phi = stats.norm.pdf
    d16 = sum(integrate.quad(lambda x: (x - c16[k]) ** 2 * phi(x), max(edges[k], -12), min(edges[k + 1], 12),
                             epsabs=0, epsrel=1e-12)[0] for k in range(len(c16)))
    assert d16 >= mse * (1 - 1e-9)
    assert d16 <= mse * (1 + (1e-4 if bits <= 5 else 2e-2))
