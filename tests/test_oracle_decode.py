"""Pins of the oracle's decode attention (CPU only)."""

import numpy as np
import pytest
import torch

from decode_attention_rope_amd import synth
from oracle import allocate, decode, energy, layout, quantize, rope


def _tiny_dequantized():
    wl = synth.TINY
    k = synth.keys(wl, 0, 0, 0, 0, 256)
    v = synth.values(wl, 0, 0, 0, 0, 256)
    bank, rv = synth.rotation_bank(64), synth.rotation_v(64)
    lay = layout.build(allocate.greedy(energy.block_energy(k), wl.budget))
    kh = quantize.dequantize_keys(*quantize.quantize_keys(k, lay, bank), lay, bank)
    vh = quantize.dequantize_values(*quantize.quantize_values(v, rv, 3), rv, 3)
    return wl, kh, vh


def test_matches_torch_sdpa_on_dequantized_cache():
    wl, kh, vh = _tiny_dequantized()
    q = synth.queries(wl, 0, 0)
    out, logits = decode.decode_head_group(q, 256, wl.theta, kh, vh)
    qr = torch.tensor(rope.apply(q, 256, wl.theta))[None, :, None, :]          # [1, H, 1, d]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qr, torch.tensor(kh)[None, None], torch.tensor(vh)[None, None])
    np.testing.assert_allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(logits[0], (kh @ rope.apply(q[0], 256, wl.theta)) / 8.0, rtol=1e-12)


def test_logits_are_block_sums_over_relative_position():
    """RoPE logit of a pre-RoPE key cached at position n equals the block-sum at relative offset n - m."""
    rng = np.random.default_rng(2)
    d, base, m = 64, 1e4, 300
    q = rng.standard_normal((1, d))
    kpre = rng.standard_normal((40, d))
    pos = np.arange(40) * 7
    kpost = rope.apply(kpre, pos, base)
    _, logits = decode.decode_head_group(q, m, base, kpost, np.zeros((40, d)), scale=1.0)
    theta = np.power(base, -2.0 * np.arange(d // 2) / d)
    qc = q[0, :32] + 1j * q[0, 32:]
    kc = kpre[:, :32] + 1j * kpre[:, 32:]
    ref = np.real(np.conj(qc)[None] * kc * np.exp(1j * (pos[:, None] - m) * theta[None])).sum(1)
    np.testing.assert_allclose(logits[0], ref, rtol=1e-10, atol=1e-10)


def test_degenerate_cases():
    rng = np.random.default_rng(3)
    d = 32
    v = rng.standard_normal((1, d))
    out, _ = decode.decode_head_group(rng.standard_normal((2, d)), 5, 1e4, rng.standard_normal((1, d)), v)
    np.testing.assert_allclose(out, np.repeat(v, 2, 0), rtol=1e-15)
    vs = rng.standard_normal((10, d))
    out, _ = decode.decode_head_group(rng.standard_normal((1, d)), 5, 1e4, np.zeros((10, d)), vs)
    np.testing.assert_allclose(out[0], vs.mean(0), rtol=1e-12)
    out, logits = decode.decode_head_group(rng.standard_normal((1, d)), 5, 1e4, np.zeros((0, d)), np.zeros((0, d)))
    assert logits.shape == (1, 0) and not out.any()


def test_softmax_shift_invariance_and_large_logits():
    rng = np.random.default_rng(4)
    d = 16
    k = rng.standard_normal((50, d)) * 40
    v = rng.standard_normal((50, d))
    q = rng.standard_normal((1, d)) * 40
    out, s = decode.decode_head_group(q, 0, 0.0, k, v)
    p = np.exp(s[0] - s[0].max())
    np.testing.assert_allclose(out[0], (p / p.sum()) @ v, rtol=1e-12)
    assert np.isfinite(out).all()
