"""Greedy integer bit-width allocation by marginal gain (oracle).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: Block-GTQ
greedily allocates integer bit widths to RoPE blocks by marginal gain, giving
more bits to high-energy blocks, under K/V bit budgets matched to the uniform
TQ-MSE baseline ("b/dim", KxVy).

Readings (the pages give no formula):

* Budget: Kx means x bits per coordinate on average, so the widths b_j
  (bits per coordinate of block j) satisfy sum_j b_j = B = x * d/2 exactly.
* Distortion model: coding a block at b bits costs E_j * D(b), with D(b) the
  MSE of the b-bit Gaussian Lloyd-Max quantizer (the per-coordinate model of
  TQ-MSE), taken as fl32(D(b)) with D(0) = 1.
* Marginal gain of one more bit for block j: E_j * (D(b_j) - D(b_j + 1)),
  the bracket evaluated in fp64 from the fp32 values, the product in fp64.
* Greedy: start every block at b_min and make B - n*b_min single-bit
  increments, each to the block of largest gain among blocks below b_max;
  equal gains go to the lowest block index.

Two further statements of the same allocation serve as pins: the sort-based
form (all candidate increments ranked at once, valid because D(b) - D(b+1)
strictly decreases in b) and exhaustive search over all width vectors.
"""

from __future__ import annotations

import itertools

import numpy as np

from .codebook import distortion32, B_MAX


class BudgetError(ValueError):
    pass


def _check(n: int, budget: int, b_min: int, b_max: int) -> None:
    if not (0 <= b_min <= b_max <= B_MAX):
        raise BudgetError("need 0 <= b_min <= b_max <= 8")
    if not (n * b_min <= budget <= n * b_max):
        raise BudgetError(f"budget {budget} infeasible for {n} blocks in [{b_min}, {b_max}]")


def gain_table() -> np.ndarray:
    """D(b) - D(b+1) for b = 0..B_MAX-1 (fp64, from the fp32 distortions)."""
    d = distortion32()
    return d[:-1] - d[1:]


def greedy(energy, budget: int, b_min: int = 0, b_max: int = B_MAX) -> np.ndarray:
    """Widths (int) for one head's block energies, by the greedy rule."""
    e = [float(x) for x in np.asarray(energy, dtype=np.float64)]
    n = len(e)
    _check(n, budget, b_min, b_max)
    dgain = gain_table()
    widths = [b_min] * n
    for _ in range(budget - n * b_min):
        best_j, best_g = -1, None
        for j in range(n):
            if widths[j] >= b_max:
                continue
            g = e[j] * float(dgain[widths[j]])
            if best_g is None or g > best_g:       # strict: ties keep the lower j
                best_j, best_g = j, g
        widths[best_j] += 1
    return np.array(widths, dtype=np.int64)


def sort_based(energy, budget: int, b_min: int = 0, b_max: int = B_MAX) -> np.ndarray:
    """Same allocation as ``greedy``: rank every (block, level) increment at once."""
    e = np.asarray(energy, dtype=np.float64)
    n = e.shape[0]
    _check(n, budget, b_min, b_max)
    dgain = gain_table()
    cands = []
    for j in range(n):
        for b in range(b_min, b_max):
            cands.append((-(float(e[j]) * float(dgain[b])), j, b))
    cands.sort()                                   # gain desc, then block asc, then level asc
    widths = np.full(n, b_min, dtype=np.int64)
    for _, j, _ in cands[: budget - n * b_min]:
        widths[j] += 1
    return widths


def objective(energy, widths) -> float:
    """sum_j E_j * D(b_j) in fp64, ascending j."""
    d = distortion32()
    total = 0.0
    for e, b in zip(np.asarray(energy, dtype=np.float64), widths):
        total += float(e) * float(d[int(b)])
    return total


def brute_force(energy, budget: int, b_min: int = 0, b_max: int = B_MAX):
    """All minimisers of the objective over width vectors with sum = budget (small n only)."""
    e = np.asarray(energy, dtype=np.float64)
    n = e.shape[0]
    _check(n, budget, b_min, b_max)
    if n > 8:
        raise ValueError("brute force is for tiny block counts")
    best, arg = None, []
    for w in itertools.product(range(b_min, b_max + 1), repeat=n):
        if sum(w) != budget:
            continue
        v = objective(e, w)
        if best is None or v < best:
            best, arg = v, [w]
        elif v == best:
            arg.append(w)
    return best, [np.array(w, dtype=np.int64) for w in arg]
