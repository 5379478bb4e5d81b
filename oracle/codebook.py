"""Gaussian Lloyd-Max codebooks for TurboQuant-MSE (oracle, fp64).

The pages name TurboQuant-MSE (TQ-MSE) as the quantizer Block-GTQ is built on
(RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract, the sentence
introducing Block-GTQ) but do not define it.  Reading used here (from the
TurboQuant paper, outside the pages): after a random rotation every coordinate
of a unit vector in R^m is close to N(0, 1/m), and each coordinate is coded
with the b-bit minimum-MSE (Lloyd-Max) scalar quantizer of that Gaussian.  The
codebook is stored for N(0, 1); the 1/sqrt(m) scale is applied separately.

The Lloyd-Max conditions for N = 2^b cells with thresholds t_1 < ... < t_{N-1}
(t_0 = -inf, t_N = +inf):

    c_k = E[X | t_{k-1} < X < t_k]            (centroid condition)
    t_k = (c_k + c_{k+1}) / 2                  (nearest-neighbour condition)

They are solved here by Newton's method on the thresholds, started from the
Panter-Dite companding guess t_k = sqrt(3) * Phi^{-1}(k/N).  The tables are
then made exactly antisymmetric and rounded to fp32: the quantizer compares
against the fp32 decision levels, and reconstruction uses the fp32 centroids
(the pages fix no precision for the codebook; levels16 gives the centroids
rounded once more to fp16, which differ by at most 2^-11 relative).  D(b) is the MSE of
the b-bit quantizer of N(0, 1); D(0) = 1 (a coordinate coded with zero bits is
reconstructed as 0).  The allocator uses fl32(D(b)).
"""

from __future__ import annotations

import math
from functools import lru_cache

import numpy as np
from scipy.special import ndtri

B_MAX = 8
_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _pdf(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _mass(a: float, b: float) -> float:
    """P(a < X < b) for X ~ N(0, 1), written to avoid cancellation in the tails."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / _SQRT2) - math.erfc(b / _SQRT2))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / _SQRT2) - math.erfc(-a / _SQRT2))
    return 0.5 * (math.erf(b / _SQRT2) - math.erf(a / _SQRT2))


def _centroid(a: float, b: float) -> tuple[float, float]:
    """(E[X | a < X < b], P(a < X < b)) for X ~ N(0, 1)."""
    p = _mass(a, b)
    return (_pdf(a) - _pdf(b)) / p, p


@lru_cache(maxsize=None)
def solve(bits: int) -> tuple[np.ndarray, np.ndarray, float]:
    """fp64 (thresholds[N-1], centroids[N], mse) of the b-bit Gaussian Lloyd-Max quantizer."""
    if not 1 <= bits <= B_MAX:
        raise ValueError(f"bits must be in 1..{B_MAX}")
    n = 1 << bits
    t = math.sqrt(3.0) * ndtri(np.arange(1, n) / n)
    for _ in range(200):
        edges = np.concatenate(([-math.inf], t, [math.inf]))
        c = np.empty(n)
        p = np.empty(n)
        for k in range(n):
            c[k], p[k] = _centroid(edges[k], edges[k + 1])
        # residual F_k = t_k - (c_k + c_{k+1}) / 2 and its tridiagonal Jacobian
        f = t - 0.5 * (c[:-1] + c[1:])
        diag = np.empty(n - 1)
        lower = np.zeros(n - 1)   # dF_k / dt_{k-1}
        upper = np.zeros(n - 1)   # dF_k / dt_{k+1}
        for k in range(n - 1):
            tk = t[k]
            # cell k (0-based) is (edges[k], edges[k+1]) = (t_{k-1}, t_k)
            dck_dtk = _pdf(tk) * (tk - c[k]) / p[k]
            dck1_dtk = _pdf(tk) * (c[k + 1] - tk) / p[k + 1]
            diag[k] = 1.0 - 0.5 * (dck_dtk + dck1_dtk)
            if k > 0:
                a = t[k - 1]
                lower[k] = -0.5 * _pdf(a) * (c[k] - a) / p[k]
            if k < n - 2:
                b = t[k + 1]
                upper[k] = -0.5 * _pdf(b) * (b - c[k + 1]) / p[k + 1]
        jac = np.diag(diag) + np.diag(lower[1:], -1) + np.diag(upper[:-1], 1)
        step = np.linalg.solve(jac, f)
        t = t - step
        if np.max(np.abs(step)) < 1e-15:
            break
    # exact antisymmetry: t_{N/2} = 0 and t_{N/2+i} = -t_{N/2-i}
    t = 0.5 * (t - t[::-1])
    t[n // 2 - 1] = 0.0
    edges = np.concatenate(([-math.inf], t, [math.inf]))
    c = np.empty(n)
    p = np.empty(n)
    for k in range(n // 2, n):
        c[k], p[k] = _centroid(edges[k], edges[k + 1])
    c[: n // 2] = -c[n // 2:][::-1]
    p[: n // 2] = p[n // 2:][::-1]
    mse = 1.0 - float(np.sum(c * c * p))
    return t, c, mse


def thresholds32(bits: int) -> np.ndarray:
    """fp32 thresholds T_b[0..2^b-2] (ascending); a code is the count of T_b[k] < z."""
    return solve(bits)[0].astype(np.float32)


def centroids32(bits: int) -> np.ndarray:
    """fp32 reconstruction levels C_b[0..2^b-1] (ascending) for N(0, 1)."""
    return solve(bits)[1].astype(np.float32)


def levels16(bits: int) -> np.ndarray:
    """Reconstruction levels: the fp32 centroids rounded to fp16 (nearest-even), as fp64 values."""
    return centroids32(bits).astype(np.float16).astype(np.float64)


def distortion32() -> np.ndarray:
    """fl32(D(b)) for b = 0..B_MAX as fp64 values; D(0) = 1."""
    d = np.empty(B_MAX + 1, dtype=np.float64)
    d[0] = 1.0
    for b in range(1, B_MAX + 1):
        d[b] = float(np.float32(solve(b)[2]))
    return d
