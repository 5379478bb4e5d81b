"""Pins of the oracle's TQ-MSE quantizer and packed layout (CPU only)."""

import math
import struct

import numpy as np
import pytest

from decode_attention_rope_amd import synth
from oracle import allocate, codebook, energy, layout, pack, quantize


@pytest.fixture(scope="module")
def bank64():
    return synth.rotation_bank(64, seed=0)


def test_rotations_orthogonal():
    bank = synth.rotation_bank(32, seed=3)
    for m in range(2, 33, 2):
        r = quantize.bank_matrix(bank, m).astype(np.float64)
        np.testing.assert_allclose(r @ r.T, np.eye(m), atol=2e-6)
    rv = synth.rotation_v(128, seed=3).astype(np.float64)
    np.testing.assert_allclose(rv @ rv.T, np.eye(128), atol=2e-6)
    assert quantize.bank_offset(2) == 0 and quantize.bank_offset(6) == 4 + 16
    assert bank.shape[0] == sum(m * m for m in range(2, 33, 2))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_uniform_widths_reduce_to_plain_tq_mse(bits, bank64):
    """All blocks at one width: one group of m = d, codes = nearest centroid of the rotated, rescaled key."""
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    lay = layout.build(np.full(32, bits))
    codes, norms = quantize.quantize_keys(x, lay, bank64)
    xs = x[:, lay.perm].astype(np.float64)
    rot = quantize.bank_matrix(bank64, 64).astype(np.float64)
    z = (xs @ rot.T) / np.linalg.norm(xs, axis=1, keepdims=True) * 8.0
    cen = codebook.solve(bits)[1]
    nearest = np.argmin(np.abs(z[..., None] - cen), axis=-1)
    thr = codebook.solve(bits)[0]
    near_tie = np.min(np.abs(z[..., None] - thr), axis=-1) < 1e-5
    assert np.all((codes == nearest) | near_tie)
    assert np.mean(near_tie) < 1e-3
    np.testing.assert_allclose(norms[:, 0].astype(np.float64), np.linalg.norm(xs, axis=1), rtol=2 ** -11)


def test_norm_and_fp16_rounding():
    """Stored norms are the fp32 norm rounded to fp16 nearest-even (checked with struct's IEEE half)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((2000, 6)) * np.exp(rng.uniform(-8, 8, size=(2000, 1)))).astype(np.float32)
    lay = layout.build([3, 3, 3])
    _, norms = quantize.quantize_keys(x, lay, synth.rotation_bank(6))
    for i in range(2000):
        xs = x[i, lay.perm].astype(np.float64)
        exact = math.sqrt(math.fsum(xs * xs))
        n32 = float(np.float32(exact))
        assert abs(n32 - exact) <= 4 * 2.0 ** -24 * exact       # sequential fp32 sum + sqrt
        if n32 < 65504:
            # the norm is summed in fp32 in storage order, then rounded to IEEE half
            ss = np.float32(0)
            for v in x[i, lay.perm]:
                ss = np.float32(ss + np.float32(v * v))
            ref = struct.unpack("<e", struct.pack("<e", float(np.sqrt(ss))))[0]
            assert float(norms[i, 0]) == ref


def test_scale_sign_and_zero(bank64):
    rng = np.random.default_rng(6)
    w = allocate.greedy(rng.exponential(size=32), 96)
    lay = layout.build(w)
    x = rng.standard_normal((500, 64)).astype(np.float32)
    c, n = quantize.quantize_keys(x, lay, bank64)
    c4, n4 = quantize.quantize_keys(x * np.float32(4.0), lay, bank64)
    np.testing.assert_array_equal(c4, c)
    np.testing.assert_array_equal(n4.astype(np.float32), (n.astype(np.float32) * 4))
    cneg, _ = quantize.quantize_keys(-x, lay, bank64)
    levels = (1 << lay.width) - 1
    np.testing.assert_array_equal(cneg, levels[None, :] - c)
    cz, nz = quantize.quantize_keys(np.zeros((3, 64), np.float32), lay, bank64)
    assert not cz.any() and not nz.astype(np.float32).any()


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_empirical_mse_matches_lloyd_max(bits):
    rng = np.random.default_rng(bits + 10)
    d = 128
    x = rng.standard_normal((4000, d)).astype(np.float32)
    rv = synth.rotation_v(d, seed=1)
    c, n = quantize.quantize_values(x, rv, bits)
    xh = quantize.dequantize_values(c, n, rv, bits)
    rel = np.sum((xh - x) ** 2) / np.sum(x.astype(np.float64) ** 2)
    assert rel == pytest.approx(codebook.solve(bits)[2], rel=0.05)


def test_pack_bits_against_integer_construction():
    """Every record equals sum_p code_p << offset_p as a little-endian integer."""
    rng = np.random.default_rng(7)
    w = rng.integers(0, 9, size=48)
    lay = layout.build(w)
    codes = rng.integers(0, 1 << lay.width, size=(130, lay.d_eff))
    rec = pack.k_record_bytes(codes, lay)
    for t in range(130):
        val = 0
        for p in range(lay.d_eff):
            val |= int(codes[t, p]) << int(lay.offset[p])
        assert bytes(rec[t]) == val.to_bytes(lay.chunks * 16, "little")


@pytest.mark.parametrize("t_len,v_bits", [(1, 3), (63, 2), (64, 3), (130, 1), (200, 8)])
def test_pack_region_layout_and_round_trip(t_len, v_bits):
    rng = np.random.default_rng(t_len)
    w = allocate.greedy(rng.exponential(size=32), 3 * 32)
    lay = layout.build(w)
    d, cap = 64, 256
    kc = rng.integers(0, 1 << lay.width, size=(t_len, lay.d_eff))
    kn = rng.standard_normal((t_len, len(lay.groups))).astype(np.float16)
    vc = rng.integers(0, 1 << v_bits, size=(t_len, d))
    vn = rng.standard_normal(t_len).astype(np.float16)
    reg = pack.pack_region(kc, kn, vc, vn, lay, v_bits, cap)
    sizes = pack.region_sizes(d, lay.chunks, v_bits, cap)
    assert {k: v.size for k, v in reg.items()} == sizes
    back = pack.unpack_region(reg, lay, v_bits, t_len)
    for a, b in zip(back, (kc, kn, vc, vn)):
        np.testing.assert_array_equal(a, b)
    # spot-check addresses written out by hand
    t = t_len - 1
    tau, s = divmod(t, 64)
    rec = pack.k_record_bytes(kc[t:t + 1], lay)[0]
    c = lay.chunks - 1
    start = ((tau * lay.chunks + c) * 64 + s) * 16
    assert bytes(reg["k_codes"][start:start + 16]) == bytes(rec[16 * c:16 * c + 16])
    seg = int.from_bytes(bytes(reg["v_codes"][(tau * d + 5) * 8 * v_bits:(tau * d + 6) * 8 * v_bits]), "little")
    assert (seg >> (s * v_bits)) & ((1 << v_bits) - 1) == vc[t, 5]
    assert reg["k_norms"][(tau * 8 + 0) * 64 + s] == kn[t, 0]
    assert reg["v_norms"][tau * 64 + s] == vn[t]
    # unused slots are zero
    assert not reg["v_norms"][t_len:].astype(np.float32).any()


def test_tiny_workload_end_to_end_quantize():
    wl = synth.TINY
    k = synth.keys(wl, 0, 0, 0, 0, 256)
    w = allocate.greedy(energy.block_energy(k), wl.budget)
    lay = layout.build(w)
    c, n = quantize.quantize_keys(k, lay, synth.rotation_bank(64))
    kh = quantize.dequantize_keys(c, n, lay, synth.rotation_bank(64))
    # Block-GTQ error below uniform 3-bit TQ-MSE on a decaying energy profile
    lay_u = layout.build(np.full(32, 3))
    cu, nu = quantize.quantize_keys(k, lay_u, synth.rotation_bank(64))
    ku = quantize.dequantize_keys(cu, nu, lay_u, synth.rotation_bank(64))
    assert np.sum((kh - k) ** 2) < np.sum((ku - k) ** 2)


@pytest.mark.parametrize("levels", ["fp16", "fp32"])
def test_one_bit_reconstruction_closed_form(levels):
    """One-bit groups with identity rotations and unit norms reconstruct every coordinate as
    +-sqrt(2/pi)/sqrt(m): the 1-bit Lloyd-Max level of N(0, 1) in closed form, rounded to fp32
    ("fp32" levels) or further to fp16 ("fp16", the levels the packed cache is decoded with)."""
    d = 16
    lay = layout.build(np.array([1, 1, 1, 1, 0, 0, 1, 1]))         # one group of six blocks, m = 12
    bank = np.zeros(sum(m * m for m in range(2, d + 1, 2)), dtype=np.float32)
    for m in range(2, d + 1, 2):
        o = quantize.bank_offset(m)
        bank[o:o + m * m] = np.eye(m, dtype=np.float32).ravel()
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 2, size=(5, lay.d_eff))
    norms = np.ones((5, 1), dtype=np.float16)
    x = quantize.dequantize_keys(codes, norms, lay, bank, levels=levels)
    c = np.float32(math.sqrt(2.0 / math.pi))
    if levels == "fp16":
        c = np.float16(c)
    want = np.zeros((5, d))
    want[:, lay.perm] = np.where(codes == 1, 1.0, -1.0) * float(c) / math.sqrt(12)
    np.testing.assert_array_equal(x, want)
    v = quantize.dequantize_values(codes[:, :12], np.ones(5, dtype=np.float16), np.eye(12), 1, levels=levels)
    np.testing.assert_array_equal(v, np.where(codes[:, :12] == 1, 1.0, -1.0) * float(c) / math.sqrt(12))
    with pytest.raises(ValueError):
        quantize.dequantize_values(codes[:, :12], np.ones(5, dtype=np.float16), np.eye(12), 1, levels="bf16")
