"""Pins of the oracle's structured (Givens-layer) rotations for TQ-MSE (CPU only).

The transform is pinned to its dense matrix (a product of exact 2 x 2 rotations built in
fp64), to orthogonality, to the inverse relation of forward and transpose, to the
Lloyd-Max distortion of Gaussian inputs (textbook values) and to the distortion of the
dense Haar rotation on sparse inputs, where a structured transform that mixes badly would
show.
"""

import math
import os

import numpy as np
import pytest

from decode_attention_rope_amd import synth
from oracle import codebook, layout, quantize

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")


def _textbook_mse(bits):
    with open(GOLDEN) as f:
        for line in f:
            p = line.split()
            if len(p) == 3 and p[0] == str(bits) and p[1] == "mse":
                return float(p[2])
    raise KeyError(bits)


@pytest.fixture(scope="module")
def giv():
    return quantize.Givens(synth.givens_bank(256, seed=3))


def test_generator_format(giv):
    rec = giv.rec
    for m in range(2, 257, 2):
        first, n_layers = int(rec[m // 2 - 1, 0]), int(rec[m // 2 - 1, 1])
        assert n_layers == synth.givens_layer_count(m) and n_layers % 2 == 1
        for a, b, c, s in giv.layers(m):
            assert sorted(np.concatenate([a, b]).tolist()) == list(range(m))      # a perfect matching
            np.testing.assert_allclose(c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2, 1.0, atol=2e-7)
        assert first >= synth.GIVENS_HEADER
    assert not rec[:synth.GIVENS_HEADER, 2:].any()


@pytest.mark.parametrize("m", [2, 6, 64, 128, 256])
def test_orthogonal_and_transpose_inverts(giv, m):
    s = giv.matrix(m)
    # fp32 cos and sin leave |c^2 + s^2 - 1| <= 2^-23 per layer
    n_layers = len(giv.layers(m))
    np.testing.assert_allclose(s @ s.T, np.eye(m), atol=2 * n_layers * 2.0 ** -23)
    x = np.random.default_rng(m).standard_normal((20, m))
    np.testing.assert_allclose(quantize.givens_transpose64(quantize.givens_forward64(x, giv.layers(m)), giv.layers(m)),
                               x, atol=2 * n_layers * 2.0 ** -23 * np.abs(x).max())


@pytest.mark.parametrize("m", [2, 30, 128, 256])
def test_fp32_forward_within_rounding_of_the_dense_product(giv, m):
    x = np.random.default_rng(m + 1).standard_normal((50, m)).astype(np.float32)
    y32 = quantize.givens_forward32(x, giv.layers(m)).astype(np.float64)
    y64 = x.astype(np.float64) @ giv.matrix(m).T
    # each layer rounds two products and one sum per coordinate (relative 2^-24 each) and the
    # fp32 cos and sin are exact inputs of both: the error grows at most linearly in the layers
    n_layers = len(giv.layers(m))
    bound = 3 * n_layers * 2.0 ** -24 * np.abs(x).max() * math.sqrt(m)
    assert np.abs(y32 - y64).max() <= bound


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_distortion_matches_lloyd_max(giv, bits):
    x = np.random.default_rng(bits).standard_normal((4000, 128)).astype(np.float32)
    rv = giv                                            # the value path takes the size-128 layers
    c, n = quantize.quantize_values(x, rv, bits)
    xh = quantize.dequantize_values(c, n, rv, bits)
    rel = np.sum((xh - x) ** 2) / np.sum(x.astype(np.float64) ** 2)
    assert rel == pytest.approx(_textbook_mse(bits), rel=0.05)


@pytest.mark.parametrize("m,nz", [(128, 1), (128, 2), (24, 1)])
def test_sparse_inputs_mix_like_a_dense_rotation(giv, m, nz):
    rng = np.random.default_rng(m + nz)
    x = np.zeros((3000, m), dtype=np.float32)
    for i in range(3000):
        x[i, rng.choice(m, nz, replace=False)] = rng.standard_normal(nz)
    bank = synth.rotation_bank(m, seed=3)
    err = {}
    for name, rot in (("haar", quantize.bank_matrix(bank, m)), ("givens", giv.layers(m))):
        c, n = quantize.tq_mse(x, rot, 3)
        xh = quantize._unrotate(codebook.levels16(3)[c] / np.sqrt(m), rot) * n.astype(np.float64)[:, None]
        err[name] = np.sum((xh - x) ** 2) / np.sum(x.astype(np.float64) ** 2)
    assert err["givens"] <= 1.15 * err["haar"], err


def test_width_groups_use_their_own_size(giv):
    """A layout's width groups are rotated by the layers of their own size, in storage order."""
    rng = np.random.default_rng(5)
    widths = np.array([3] * 10 + [2] * 20 + [0] * 2)       # groups of m = 20 and m = 40, d = 64
    lay = layout.build(widths)
    k = rng.standard_normal((30, 64)).astype(np.float32)
    codes, norms = quantize.quantize_keys(k, lay, giv)
    for g, grp in enumerate(lay.groups):
        cols = lay.perm[grp.first:grp.first + grp.m]
        c, n = quantize.tq_mse(k[:, cols], giv.layers(grp.m), grp.width)
        np.testing.assert_array_equal(codes[:, grp.first:grp.first + grp.m], c)
        np.testing.assert_array_equal(norms[:, g], n)
    kh = quantize.dequantize_keys(codes, norms, lay, giv)
    dropped = np.setdiff1d(np.arange(64), lay.perm)
    assert dropped.size == 4 and not kh[:, dropped].any()             # width-0 blocks reconstruct as 0
    kept = lay.perm
    rel = np.sum((kh[:, kept] - k[:, kept]) ** 2) / np.sum(k[:, kept].astype(np.float64) ** 2)
    assert rel < 0.15
