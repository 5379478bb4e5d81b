"""Pins of the oracle's fp16 recent-key window (CPU only).

The fp16 rounding is pinned to hand-derived binary16 values (ties to even, the largest
finite value, saturation, subnormals); the window's effect on attention to torch's own
attention with torch's own fp16 conversion; the window boundary to the no-window decode.
"""

import numpy as np
import pytest
import torch

from decode_attention_rope_amd import synth
from oracle import allocate, decode, energy, layout, quantize, rope, window


def test_fp16_rounding_by_hand():
    one = 1.0
    cases = [
        (one + 2.0 ** -11, one),                      # halfway, even neighbour below
        (one + 3 * 2.0 ** -11, one + 2.0 ** -9),      # halfway, even neighbour above
        (one + 2.0 ** -11 + 2.0 ** -20, one + 2.0 ** -10),
        (65504.0, 65504.0),
        (65519.0, 65504.0),                           # below the halfway point to 65536
        (65520.0, 65504.0),                           # IEEE would give inf: saturated
        (1e9, 65504.0),
        (-1e9, -65504.0),
        (2.0 ** -24, 2.0 ** -24),                     # smallest subnormal
        (2.0 ** -25, 0.0),                            # halfway to it: even (zero)
        (3 * 2.0 ** -26, 2.0 ** -24),
        (-0.0, -0.0),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    got = window.fp16_keys(x)
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[-1])


def _tiny(t_len=256):
    wl = synth.TINY
    k = synth.keys(wl, 0, 0, 0, 0, t_len)
    v = synth.values(wl, 0, 0, 0, 0, t_len)
    bank, rv = synth.rotation_bank(64), synth.rotation_v(64)
    lay = layout.build(allocate.greedy(energy.block_energy(k), wl.budget))
    kh = quantize.dequantize_keys(*quantize.quantize_keys(k, lay, bank), lay, bank)
    vh = quantize.dequantize_values(*quantize.quantize_values(v, rv, 3), rv, 3)
    return wl, k, kh, vh


def test_window_zero_is_the_packed_decode():
    wl, k, kh, vh = _tiny()
    q = synth.queries(wl, 0, 0)
    a = window.decode_head_group(q, 255, wl.theta, kh, k, vh, 0)
    b = decode.decode_head_group(q, 255, wl.theta, kh, vh)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_whole_sequence_window_matches_torch_attention_on_fp16_keys():
    wl, k, kh, vh = _tiny()
    q = synth.queries(wl, 0, 0)
    out, logits = window.decode_head_group(q, 255, wl.theta, kh, k, vh, 4096)
    k16 = torch.tensor(k).half().double()                          # torch's own fp16 rounding
    qr = torch.tensor(rope.apply(q, 255, wl.theta))
    ref = torch.nn.functional.scaled_dot_product_attention(qr[None, :, None, :], k16[None, None],
                                                           torch.tensor(vh)[None, None])
    np.testing.assert_allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(logits, (qr @ k16.T).numpy() / 8.0, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("w", [1, 7, 64, 100])
def test_window_boundary(w):
    """Only the newest w logits move; they move to the fp16-key logits."""
    wl, k, kh, vh = _tiny()
    q = synth.queries(wl, 0, 0)
    _, lw = window.decode_head_group(q, 255, wl.theta, kh, k, vh, w)
    _, l0 = decode.decode_head_group(q, 255, wl.theta, kh, vh)
    _, l16 = decode.decode_head_group(q, 255, wl.theta, window.fp16_keys(k), vh)
    np.testing.assert_array_equal(lw[:, :256 - w], l0[:, :256 - w])
    np.testing.assert_array_equal(lw[:, 256 - w:], l16[:, 256 - w:])
    assert window.window_range(256, w) == (256 - w, 256)
    assert window.window_range(5, 0) == (5, 5) and window.window_range(5, 9) == (0, 5)


def test_ring_slots_are_distinct_and_cover_the_window():
    for t_len, w in [(10, 4), (4, 10), (130, 64), (64, 64)]:
        slots = window.ring_slots(t_len, w)
        assert len(slots) == min(t_len, w)
        assert len(set(slots.values())) == len(slots)
        assert all(0 <= v < w for v in slots.values())


def test_window_keys_cut_the_logit_error():
    """fp16 keys are far closer to the exact keys than 3-bit reconstructions (sanity of the reading)."""
    wl, k, kh, vh = _tiny()
    q = synth.queries(wl, 0, 0)
    _, exact = decode.decode_head_group(q, 255, wl.theta, k.astype(np.float64), vh)
    _, lw = window.decode_head_group(q, 255, wl.theta, kh, k, vh, 64)
    _, l0 = decode.decode_head_group(q, 255, wl.theta, kh, vh)
    e_w = np.abs(lw - exact)[:, -64:].mean()
    e_0 = np.abs(l0 - exact)[:, -64:].mean()
    assert e_w < 0.1 * e_0
