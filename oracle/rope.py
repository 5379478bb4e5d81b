"""Rotary position embedding in fp64 (oracle).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: with RoPE, the
logit a cached key contributes to splits into one term per 2-D frequency block,
and each term depends on the query-key position gap.  Block j rotates its two coordinates by the
angle pos * theta_j with theta_j = base^(-2j/d).

Readings (the pages give no layout): block j pairs coordinates (j, j + d/2)
("half" pairing, as the Llama/Qwen checkpoints do) or (2j, 2j+1)
("interleaved").  The angle pos * theta_j is formed in fp64 and reduced modulo
2*pi in fp64 before cos/sin, so positions near 2^19 keep full accuracy.
"""

from __future__ import annotations

import math

import numpy as np

HALF = 0
INTERLEAVED = 1


def block_coords(d: int, pairing: int) -> tuple[np.ndarray, np.ndarray]:
    """(first, second) coordinate index of every RoPE block j = 0..d/2-1."""
    n = d // 2
    j = np.arange(n)
    if pairing == HALF:
        return j, j + n
    if pairing == INTERLEAVED:
        return 2 * j, 2 * j + 1
    raise ValueError("pairing must be HALF (0) or INTERLEAVED (1)")


def inv_freq(d: int, base: float) -> np.ndarray:
    """theta_j = base^(-2j/d), fp64."""
    j = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / d)


def angles(pos, d: int, base: float) -> np.ndarray:
    """pos * theta_j reduced to [0, 2*pi), fp64; shape pos.shape + (d/2,)."""
    p = np.asarray(pos, dtype=np.float64)[..., None]
    return np.mod(p * inv_freq(d, base), 2.0 * math.pi)


def apply(x, pos, base: float, pairing: int = HALF) -> np.ndarray:
    """RoPE of x[..., d] at positions pos (broadcast over x's leading axes), fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a, b = block_coords(d, pairing)
    ang = angles(pos, d, base)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., a] = x[..., a] * c - x[..., b] * s
    out[..., b] = x[..., a] * s + x[..., b] * c
    return out
