"""Pins of the oracle's RoPE and block-energy score (CPU only)."""

import math

import numpy as np
import pytest

from oracle import energy, rope


def _complex_blocks(x, pairing):
    a, b = rope.block_coords(x.shape[-1], pairing)
    return x[..., a] + 1j * x[..., b]


@pytest.mark.parametrize("pairing", [rope.HALF, rope.INTERLEAVED])
def test_logit_is_sum_of_block_terms(pairing):
    """q_m . k_n after RoPE equals sum_j Re(conj(q_j) k_j e^{i (n - m) theta_j}) on pre-RoPE blocks."""
    rng = np.random.default_rng(1)
    d, base = 128, 1e4
    for m, n in [(0, 0), (5, 17), (1000, 3), (131071, 131072), (524287, 7)]:
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        lhs = rope.apply(q, m, base, pairing) @ rope.apply(k, n, base, pairing)
        theta = np.power(base, -2.0 * np.arange(d // 2) / d)
        terms = np.real(np.conj(_complex_blocks(q, pairing)) * _complex_blocks(k, pairing)
                        * np.exp(1j * (n - m) * theta))
        assert lhs == pytest.approx(terms.sum(), rel=1e-9, abs=1e-9)
        if m == n:
            assert lhs == pytest.approx(q @ k, rel=1e-12)


def test_rope_composes_and_keeps_block_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 64))
    p1, p2 = 300007, 224281
    two = rope.apply(rope.apply(x, p1, 1e6), p2, 1e6)
    one = rope.apply(x, p1 + p2, 1e6)
    np.testing.assert_allclose(two, one, rtol=0, atol=1e-9)
    a, b = rope.block_coords(64, rope.HALF)
    np.testing.assert_allclose(one[:, a] ** 2 + one[:, b] ** 2, x[:, a] ** 2 + x[:, b] ** 2, rtol=1e-12)


def test_interleaved_is_a_permutation_of_half():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(32)
    perm = np.empty(32, dtype=int)
    perm[0::2] = np.arange(16)
    perm[1::2] = np.arange(16) + 16
    np.testing.assert_allclose(rope.apply(x[perm], 77, 1e4, rope.INTERLEAVED),
                               rope.apply(x, 77, 1e4, rope.HALF)[perm], rtol=1e-14)


def test_energy_exact_on_dyadic_keys():
    k = np.zeros((1000, 8), dtype=np.float32)
    k[:, 0], k[:, 4], k[:, 1], k[:, 5] = 0.5, 1.5, -2.0, 0.25
    e = energy.block_energy(k)
    assert e.tolist() == [2.5, 4.0625, 0.0, 0.0]


@pytest.mark.parametrize("t_len", [1, 255, 256, 257, 5000])
def test_energy_within_sequential_sum_bound(t_len):
    """Against the exactly rounded sum (math.fsum) within the bound of a length-T fp64 sum."""
    rng = np.random.default_rng(t_len)
    k = (rng.standard_normal((t_len, 16)) * 3).astype(np.float32)
    e = energy.block_energy(k)
    k64 = k.astype(np.float64)
    for j in range(8):
        terms = k64[:, j] ** 2 + k64[:, j + 8] ** 2
        exact = math.fsum(terms) / t_len
        assert abs(e[j] - exact) <= (t_len + 2) * 2.0 ** -52 * exact


def test_energy_rope_invariant_and_matches_closed_form():
    rng = np.random.default_rng(4)
    t_len, d = 8192, 64
    sig = np.linspace(1.0, 0.05, d // 2)
    k = rng.standard_normal((t_len, d)) * np.concatenate([sig, sig])
    kr = rope.apply(k, np.arange(t_len), 1e4)
    e_pre, e_post = energy.block_energy(k), energy.block_energy(kr)
    np.testing.assert_allclose(e_post, e_pre, rtol=1e-12)
    # E_j = mean of sigma_j^2 * chi^2_2: expectation 2 sigma_j^2, relative std 1/sqrt(T)
    np.testing.assert_allclose(e_pre, 2 * sig ** 2, rtol=6 / math.sqrt(t_len))


def test_energy_interleaved_pairing():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((300, 16)).astype(np.float32)
    e = energy.block_energy(k, rope.INTERLEAVED)
    exact = [math.fsum(k[:, 2 * j].astype(np.float64) ** 2 + k[:, 2 * j + 1].astype(np.float64) ** 2) / 300
             for j in range(8)]
    np.testing.assert_allclose(e, exact, rtol=1e-13)
