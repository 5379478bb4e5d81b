"""Pins of the oracle's key-only logit-error diagnostic (CPU only).

The diagnostic compares the RoPE query-key logits of quantized keys with the exact ones.
Each pin below fixes a part of it against something other than the oracle itself: the
relative-position form of RoPE (complex arithmetic), a perturbed-key closed form, the case
where Block-GTQ reduces to uniform TQ-MSE, the Gaussian error model of a rotated scalar
quantizer with the textbook Lloyd-Max distortions, and the direction of the comparison the
abstract reports.
"""

import math
import os

import numpy as np
import pytest

from decode_attention_rope_amd import synth
from oracle import diagnostic, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")


def _textbook_mse(bits):
    with open(GOLDEN) as f:
        for line in f:
            p = line.split()
            if len(p) == 3 and p[0] == str(bits) and p[1] == "mse":
                return float(p[2])
    raise KeyError(bits)


@pytest.mark.parametrize("pairing", [rope.HALF, rope.INTERLEAVED])
def test_exact_logits_follow_relative_position(pairing):
    """scale * RoPE(q, m) . RoPE(k, p) = scale * Re sum_j conj(q_j) k_j exp(i (p - m) theta_j)."""
    rng = np.random.default_rng(11)
    d, base, m = 64, 1e6, 1000
    q = rng.standard_normal((3, d))
    kpre = rng.standard_normal((50, d))
    pos = np.arange(50) * 13
    a, b = rope.block_coords(d, pairing)
    kpost = rope.apply(kpre, pos, base, pairing)
    got = diagnostic.exact_logits(q, m, base, kpost, scale=0.25, pairing=pairing)
    theta = np.power(base, -2.0 * np.arange(d // 2) / d)
    qc = q[:, a] + 1j * q[:, b]
    kc = kpre[:, a] + 1j * kpre[:, b]
    ref = 0.25 * np.real(np.einsum("hj,tj->ht", np.conj(qc), kc * np.exp(1j * (pos[:, None] - m) * theta[None])))
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_perturbed_key_closed_form():
    """Adding delta to coordinate c of a fraction f of the keys gives MAE = scale |delta| |q'_c| f."""
    rng = np.random.default_rng(12)
    d, base, pos, c, delta = 128, 1e4, 77, 37, 0.125
    q = rng.standard_normal((4, d))
    k = rng.standard_normal((40, d))
    kh = k.copy()
    kh[::4, c] += delta                               # 10 of 40 tokens
    got = diagnostic.logit_mae(q, pos, base, k, kh, scale=0.5)
    # q'_c from the block rotation written out: c is the first coordinate of block c (half pairing)
    ang = pos * base ** (-2.0 * c / d) % (2 * math.pi)
    qc = q[:, c] * math.cos(ang) - q[:, c + d // 2] * math.sin(ang)
    np.testing.assert_allclose(got, 0.5 * delta * np.abs(qc) * 0.25, rtol=1e-12)
    assert not diagnostic.logit_mae(q, pos, base, k, k).any()
    assert diagnostic.logit_mae(q, pos, base, k[:0], k[:0]).shape == (4,)


@pytest.mark.parametrize("bits", [2, 3])
def test_flat_energy_block_gtq_is_uniform(bits):
    """Blocks of (near) equal energy get equal widths, so both methods give the same logits."""
    rng = np.random.default_rng(13 + bits)
    d = 64
    k = rng.standard_normal((1024, d)).astype(np.float32)
    q = rng.standard_normal((2, d))
    bank = synth.rotation_bank(d, seed=2)
    np.testing.assert_array_equal(diagnostic.block_gtq_widths(k, bits), diagnostic.uniform_widths(d, bits))
    u = diagnostic.k_only_mae(q, 1024, 1e4, k, bits, bank, "uniform")
    g = diagnostic.k_only_mae(q, 1024, 1e4, k, bits, bank, "block_gtq")
    np.testing.assert_array_equal(u, g)


@pytest.mark.parametrize("bits", [2, 3])
def test_uniform_error_matches_the_gaussian_model(bits):
    """Rotated scalar quantization leaves q'.(k - k_hat) ~ N(0, |q'|^2 |k|^2 D(b) / d), so
    E|error| = sqrt(2/pi) * scale * |q'| * |k| * sqrt(D(b)/d), D(b) the textbook Lloyd-Max MSE."""
    rng = np.random.default_rng(20 + bits)
    d, t_len, base, pos = 128, 4096, 1e4, 4096
    k = rng.standard_normal((t_len, d)).astype(np.float32)
    q = rng.standard_normal((3, d))
    bank = synth.rotation_bank(d, seed=4)
    got = diagnostic.k_only_mae(q, pos, base, k, bits, bank, "uniform", scale=1.0)
    qn = np.linalg.norm(q, axis=1)                    # RoPE keeps the norm
    kn = np.linalg.norm(k.astype(np.float64), axis=1).mean()
    model = math.sqrt(2 / math.pi) * qn * kn * math.sqrt(_textbook_mse(bits) / d)
    np.testing.assert_allclose(got, model, rtol=0.08)


def _panel_case(profile, d, layer):
    wl = synth.Workload("diag_pin", 71, d=d, h_q=4, h_kv=1, theta=1e6, layers=2, seq_lens=(2048,), k_bits=3,
                        v_bits=3, key_dtype="f32", profile=profile, outlier_blocks=2)
    return wl, synth.keys(wl, 0, layer, 0, 0, 2048), synth.queries(wl, 0, layer)


@pytest.mark.parametrize("profile", ["decay", "decay_jitter", "loguniform"])
@pytest.mark.parametrize("bits", [2, 3])
def test_block_gtq_beats_uniform_on_skewed_profiles(profile, bits):
    """The abstract's direction: at a matched budget the greedy widths lower the key-only
    logit error on skewed block energies (magnitude not pinned)."""
    bank = synth.rotation_bank(128, seed=5)
    for layer in range(2):
        wl, k, q = _panel_case(profile, 128, layer)
        u = diagnostic.k_only_mae(q, 2047, wl.theta, k, bits, bank, "uniform")
        g = diagnostic.k_only_mae(q, 2047, wl.theta, k, bits, bank, "block_gtq")
        assert g.mean() < u.mean(), (profile, bits, layer, g.mean(), u.mean())


def test_more_bits_lower_error():
    bank = synth.rotation_bank(128, seed=5)
    wl, k, q = _panel_case("decay_jitter", 128, 0)
    for method in ("uniform", "block_gtq"):
        e = [diagnostic.k_only_mae(q, 2047, wl.theta, k, b, bank, method).mean() for b in (2, 3, 4)]
        assert e[0] > e[1] > e[2], (method, e)
