"""Pins of the oracle's greedy bit allocation and width-group layout (CPU only)."""

import numpy as np
import pytest

from decode_attention_rope_amd import synth
from oracle import allocate, energy, layout


def _cases(n, seed, count):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        kind = rng.integers(4)
        if kind == 0:
            e = rng.exponential(size=n)
        elif kind == 1:
            e = np.exp(rng.uniform(-7, 0, size=n))
        elif kind == 2:
            e = rng.integers(0, 3, size=n).astype(float)        # many exact ties, zeros
        else:
            e = np.full(n, 0.37)
        b_min = int(rng.integers(0, 3))
        b_max = int(rng.integers(max(b_min, 1), 9))
        budget = int(rng.integers(n * b_min, n * b_max + 1))
        yield e, budget, b_min, b_max


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_greedy_is_optimal_by_brute_force(n):
    for e, budget, b_min, b_max in _cases(n, 100 + n, 40 if n < 6 else 12):
        g = allocate.greedy(e, budget, b_min, b_max)
        best, args = allocate.brute_force(e, budget, b_min, b_max)
        assert allocate.objective(e, g) == pytest.approx(best, rel=1e-14, abs=1e-300)
        if len(args) == 1:
            np.testing.assert_array_equal(g, args[0])


def test_greedy_equals_sort_based():
    for n in (7, 32, 64):
        for e, budget, b_min, b_max in _cases(n, 200 + n, 25):
            np.testing.assert_array_equal(allocate.greedy(e, budget, b_min, b_max),
                                          allocate.sort_based(e, budget, b_min, b_max))


def test_budget_and_bounds():
    for e, budget, b_min, b_max in _cases(64, 7, 30):
        w = allocate.greedy(e, budget, b_min, b_max)
        assert int(w.sum()) == budget
        assert w.min() >= b_min and w.max() <= b_max


@pytest.mark.parametrize("x", [0, 1, 2, 3, 4, 8])
def test_equal_energies_give_uniform_widths(x):
    n = 64
    np.testing.assert_array_equal(allocate.greedy(np.full(n, 0.25), x * n), np.full(n, x))
    w = allocate.greedy(np.full(n, 0.25), x * n + 5) if x < 8 else None
    if w is not None:
        np.testing.assert_array_equal(w, np.r_[np.full(5, x + 1), np.full(n - 5, x)])


def test_higher_energy_gets_at_least_as_many_bits():
    rng = np.random.default_rng(9)
    for _ in range(50):
        e = rng.exponential(size=32)
        w = allocate.greedy(e, int(rng.integers(0, 257)))
        for i in range(32):
            for j in range(32):
                if e[i] > e[j] and w[j] < 8:
                    assert w[i] >= w[j]


def test_infeasible_budget_raises():
    with pytest.raises(allocate.BudgetError):
        allocate.greedy(np.ones(4), 33)
    with pytest.raises(allocate.BudgetError):
        allocate.greedy(np.ones(4), 3, b_min=1)
    with pytest.raises(allocate.BudgetError):
        allocate.greedy(np.ones(4), 4, b_min=2, b_max=1)


def test_tiny_workload_six_block_subcases():
    """Blocks 0-5 of the 256-token tiny workload at 3 b/dim, and the two outlier blocks plus four others."""
    wl = synth.TINY
    e = energy.block_energy(synth.keys(wl, 0, 0, 0, 0, 256))
    out = np.flatnonzero(synth.sigma(wl, 0, 0, 0) > 1.0)
    for idx in (np.arange(6), np.r_[out, [i for i in range(32) if i not in out][:4]]):
        sub = e[idx]
        g = allocate.greedy(sub, 18)
        best, args = allocate.brute_force(sub, 18)
        assert len(args) == 1
        np.testing.assert_array_equal(g, args[0])
    full = allocate.greedy(e, wl.budget)
    others = np.setdiff1d(np.arange(32), out)
    assert int(full.sum()) == 96 and full[out].min() >= full[others].max()


def test_layout_structure():
    rng = np.random.default_rng(11)
    for _ in range(20):
        n = int(rng.integers(1, 129))
        w = rng.integers(0, 9, size=n)
        lay = layout.build(w)
        d = 2 * n
        kept = np.flatnonzero(w > 0)
        assert sorted(lay.perm.tolist()) == sorted(np.r_[kept, kept + n].tolist())
        assert lay.code_bits == 2 * int(w.sum())
        assert lay.chunks == -(-lay.code_bits // 128)
        assert [g.width for g in lay.groups] == sorted({int(x) for x in w if x > 0}, reverse=True)
        assert np.all(np.diff(lay.width) <= 0)
        np.testing.assert_array_equal(lay.offset, np.r_[0, np.cumsum(lay.width)[:-1]] if lay.d_eff else [])
        for g in lay.groups:
            assert g.m == 2 * len(g.blocks) and list(g.blocks) == sorted(g.blocks)
            seg = lay.perm[g.first:g.first + g.m]
            assert seg.tolist() == [c for j in g.blocks for c in (j, j + n)]
        assert lay.d == d
