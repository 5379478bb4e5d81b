"""Oracle-side expectations shared by the GPU parity tests (calls only oracle/ and synth)."""

import numpy as np

from oracle import allocate, decode, energy, layout, pack, quantize, rope

TOL = 2e-3  # normwise max relative error for logits and outputs


def head_reference(k, v, budget, v_bits, bank, rv, capacity, pairing=rope.HALF, b_min=0, b_max=8):
    """Everything the oracle says about one (sequence, KV head) cache region."""
    e = energy.block_energy(k, pairing)
    w = allocate.greedy(e, budget, b_min, b_max)
    lay = layout.build(w, pairing)
    kc, kn = quantize.quantize_keys(k, lay, bank)
    vc, vn = quantize.quantize_values(v, rv, v_bits)
    return {
        "energy": e, "widths": w, "layout": lay,
        "region": pack.pack_region(kc, kn, vc, vn, lay, v_bits, capacity),
        "k_hat": quantize.dequantize_keys(kc, kn, lay, bank),
        "v_hat": quantize.dequantize_values(vc, vn, rv, v_bits),
    }


def decode_reference(q_group, pos, theta, ref, scale=None, pairing=rope.HALF):
    return decode.decode_head_group(q_group, pos, theta, ref["k_hat"], ref["v_hat"], scale=scale, pairing=pairing)


def rel_err(got, want):
    """Per row: max |got - want| / max |want|."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return np.max(np.abs(got - want), axis=-1) / np.max(np.abs(want), axis=-1)


def assert_region_equal(got: dict, want: dict, t_len: int, lay, v_bits: int, d: int):
    """Bit-exact comparison of every slot below t_len (unused slots are unspecified)."""
    tiles = -(-t_len // pack.TILE)
    used = (np.arange(tiles * pack.TILE) < t_len).reshape(tiles, pack.TILE)
    ch, ng = lay.chunks, len(lay.groups)
    if ch:
        kc_g = got["k_codes"].reshape(-1, ch, pack.TILE, 16)[:tiles].transpose(0, 2, 1, 3)
        kc_w = want["k_codes"].reshape(-1, ch, pack.TILE, 16)[:tiles].transpose(0, 2, 1, 3)
        np.testing.assert_array_equal(kc_g[used], kc_w[used], err_msg="k_codes")
    kn_g = got["k_norms"].view(np.uint16).reshape(-1, pack.MAX_GROUPS, pack.TILE)[:tiles, :ng].transpose(0, 2, 1)
    kn_w = want["k_norms"].view(np.uint16).reshape(-1, pack.MAX_GROUPS, pack.TILE)[:tiles, :ng].transpose(0, 2, 1)
    np.testing.assert_array_equal(kn_g[used], kn_w[used], err_msg="k_norms")
    vn_g = got["v_norms"].view(np.uint16).reshape(-1, pack.TILE)[:tiles]
    vn_w = want["v_norms"].view(np.uint16).reshape(-1, pack.TILE)[:tiles]
    np.testing.assert_array_equal(vn_g[used], vn_w[used], err_msg="v_norms")
    # V segments: every bit of a used slot
    bits_g = np.unpackbits(got["v_codes"].reshape(-1, d, 8 * v_bits)[:tiles], axis=2, bitorder="little")
    bits_w = np.unpackbits(want["v_codes"].reshape(-1, d, 8 * v_bits)[:tiles], axis=2, bitorder="little")
    bits_g = bits_g.reshape(tiles, d, pack.TILE, v_bits).transpose(0, 2, 1, 3)
    bits_w = bits_w.reshape(tiles, d, pack.TILE, v_bits).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(bits_g[used], bits_w[used], err_msg="v_codes")
