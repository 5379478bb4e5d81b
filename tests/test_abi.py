"""The C-ABI library loads, exports every declared call, and validates on the host (CPU only)."""

import ctypes

import numpy as np
import pytest

from decode_attention_rope_amd import bgtq
from oracle import codebook, pack

FAKE = 0x10000  # never dereferenced: every case below fails validation before any HIP call


def test_exports_every_declared_symbol():
    names = bgtq.header_functions()
    assert {"bgtq_block_energy", "bgtq_allocate_bits", "bgtq_quantize_append", "bgtq_decode_attention"} <= set(names)
    lib = bgtq.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(bgtq._SIGNATURES), "binding and header disagree"


@pytest.mark.parametrize("bits", range(0, 9))
def test_library_tables_equal_oracle_tables(bits):
    """The library's own Lloyd-Max solve (C++) agrees bit for bit with the oracle's (numpy)."""
    thr, cen, dist = bgtq.codebook(bits)
    assert dist == codebook.distortion32()[bits]
    if bits:
        np.testing.assert_array_equal(thr, codebook.thresholds32(bits))
        np.testing.assert_array_equal(cen, codebook.centroids32(bits))


@pytest.mark.parametrize("d,ksum,vb,cap", [(64, 96, 3, 256), (128, 192, 3, 131136), (128, 128, 2, 64),
                                           (256, 1024, 8, 128), (128, 0, 1, 64)])
def test_cache_sizes_match_layout(d, ksum, vb, cap):
    total, parts = bgtq.cache_bytes(2, 3, d, ksum, vb, cap)
    chunks = -(-2 * ksum // 128)
    ref = pack.region_sizes(d, chunks, vb, cap)
    per = [ref["k_codes"], ref["k_norms"] * 2, ref["v_codes"], ref["v_norms"] * 2]
    assert list(parts) == [6 * x for x in per] and total == sum(parts)


def test_invalid_geometry_sizes_are_zero():
    lib = bgtq.lib()
    assert lib.bgtq_cache_bytes(1, 1, 63, 96, 3, 256, None) == 0
    assert lib.bgtq_cache_bytes(1, 1, 64, 96, 3, 100, None) == 0
    assert lib.bgtq_cache_bytes(1, 1, 64, 96, 9, 256, None) == 0
    assert lib.bgtq_cache_bytes(1, 1, 64, 257, 3, 256, None) == 0
    assert lib.bgtq_decode_workspace_bytes(1, 16, 2, 128, 131072) > 0


def test_energy_validation():
    lib = bgtq.lib()
    ws = 1 << 20
    assert lib.bgtq_block_energy(None, 0, 1, 10, 64, 640, 64, 0, FAKE, FAKE, ws, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_block_energy(FAKE, 0, 1, 10, 63, 630, 63, 0, FAKE, FAKE, ws, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_block_energy(FAKE, 0, 1, 0, 64, 640, 64, 0, FAKE, FAKE, ws, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_block_energy(FAKE, 7, 1, 10, 64, 640, 64, 0, FAKE, FAKE, ws, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_block_energy(FAKE, 0, 1, 10, 64, 640, 32, 0, FAKE, FAKE, ws, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_block_energy(FAKE, 0, 1, 10, 64, 640, 64, 0, FAKE, FAKE, 8, None) == bgtq.ERR_WORKSPACE
    assert lib.bgtq_block_energy(FAKE, 0, 1, 10, 64, 640, 64, 0, FAKE, None, ws, None) == bgtq.ERR_WORKSPACE
    assert b"workspace" in lib.bgtq_last_error()


def test_allocate_validation():
    lib = bgtq.lib()
    assert lib.bgtq_allocate_bits(None, 1, 64, 96, 0, 8, 0, FAKE, FAKE, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_allocate_bits(FAKE, 1, 64, 257, 0, 8, 0, FAKE, FAKE, None) == bgtq.ERR_BUDGET
    assert lib.bgtq_allocate_bits(FAKE, 1, 64, 31, 1, 8, 0, FAKE, FAKE, None) == bgtq.ERR_BUDGET
    assert lib.bgtq_allocate_bits(FAKE, 1, 64, 96, 0, 9, 0, FAKE, FAKE, None) == bgtq.ERR_BUDGET
    assert lib.bgtq_allocate_bits(FAKE, 1, 64, 96, 4, 3, 0, FAKE, FAKE, None) == bgtq.ERR_BUDGET
    assert lib.bgtq_allocate_bits(FAKE, 0, 64, 96, 0, 8, 0, FAKE, FAKE, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_allocate_bits(FAKE, 1, 64, 96, 0, 8, 5, FAKE, FAKE, None) == bgtq.ERR_INVALID_ARG


def _desc(**over):
    base = dict(batch=1, n_kv_heads=2, head_dim=128, k_width_sum=192, v_bits=3, capacity=256, pairing=0,
                k_codes=FAKE, k_norms=FAKE, v_codes=FAKE, v_norms=FAKE, lengths=FAKE, widths=FAKE,
                layouts=FAKE, status=None, window=0, k_window=None)
    base.update(over)
    return bgtq.CacheDesc(*[base[f] for f, _ in bgtq.CacheDesc._fields_])


def _quantizer(d=128):
    return bgtq.Quantizer(FAKE, FAKE, FAKE, FAKE, d)


def test_append_validation():
    lib = bgtq.lib()

    def call(desc, qz=None, n_new=1, seq_begin=0, n_seqs=1, st=(1, 1, 128), dtype=0, keys=FAKE):
        qz = qz or _quantizer()
        return lib.bgtq_quantize_append(ctypes.byref(qz), ctypes.byref(desc), seq_begin, n_seqs, keys, FAKE,
                                        dtype, n_new, *(st[0] * 1000, st[1] * 300, st[2]), None)

    assert call(_desc(capacity=100)) == bgtq.ERR_INVALID_ARG
    assert call(_desc(v_bits=0)) == bgtq.ERR_INVALID_ARG
    assert call(_desc(k_width_sum=1025)) == bgtq.ERR_BUDGET
    assert call(_desc(lengths=None)) == bgtq.ERR_INVALID_ARG
    assert call(_desc(layouts=None)) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), qz=_quantizer(64)) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), n_new=0) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), n_new=257) == bgtq.ERR_CAPACITY
    assert call(_desc(), seq_begin=1) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), st=(1, 1, 64)) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), dtype=3) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), keys=None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_quantize_append(None, ctypes.byref(_desc()), 0, 1, FAKE, FAKE, 0, 1, 1, 1, 128,
                                    None) == bgtq.ERR_INVALID_ARG


def test_rotation_helpers_validation():
    lib = bgtq.lib()
    assert lib.bgtq_rotation_bank_floats(128) == sum(m * m for m in range(2, 129, 2))
    assert lib.bgtq_rotation_bank_floats(64) == sum(m * m for m in range(2, 65, 2))
    assert lib.bgtq_rotation_bank_floats(63) == 0 and lib.bgtq_rotation_bank_floats(258) == 0
    assert lib.bgtq_transpose_rotations(None, FAKE, 128, FAKE, FAKE, None) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_transpose_rotations(FAKE, FAKE, 127, FAKE, FAKE, None) == bgtq.ERR_INVALID_ARG


def test_quantizer_without_transposed_rotations_is_rejected():
    lib = bgtq.lib()
    qz = bgtq.Quantizer(FAKE, FAKE, None, FAKE, 128)
    assert lib.bgtq_quantize_append(ctypes.byref(qz), ctypes.byref(_desc()), 0, 1, FAKE, FAKE, 0, 1, 1000, 300,
                                    128, None) == bgtq.ERR_INVALID_ARG


def test_decode_validation():
    lib = bgtq.lib()
    need = lib.bgtq_decode_workspace_bytes(1, 16, 2, 128, 256)

    def call(desc, n_q=16, ws=need, qz=None, scale=0.088, d=None):
        qz = qz or _quantizer()
        return lib.bgtq_decode_attention(ctypes.byref(qz), ctypes.byref(desc), n_q, FAKE, 0, None, 1e6, scale,
                                         FAKE, None, FAKE, ws, None)

    assert call(_desc(), n_q=15) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), n_q=1) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), n_q=34) == bgtq.ERR_UNSUPPORTED
    assert call(_desc(head_dim=96), qz=_quantizer(96)) == bgtq.ERR_UNSUPPORTED
    assert call(_desc(), ws=need - 1) == bgtq.ERR_WORKSPACE
    assert call(_desc(), scale=0.0) == bgtq.ERR_INVALID_ARG
    assert call(_desc(k_norms=None)) == bgtq.ERR_INVALID_ARG


def test_decode_step_validation():
    lib = bgtq.lib()
    need = lib.bgtq_decode_workspace_bytes(1, 16, 2, 128, 256)

    def call(desc, n_q=16, ws=need, qz=None, scale=0.088, kv=FAKE, kv_dtype=0, stride_head=128):
        qz = qz or _quantizer()
        return lib.bgtq_decode_step(ctypes.byref(qz), ctypes.byref(desc), n_q, FAKE, 0, kv, kv, kv_dtype,
                                    256, stride_head, 1e6, scale, FAKE, None, FAKE, ws, None)

    assert call(_desc(), n_q=15) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), n_q=34) == bgtq.ERR_UNSUPPORTED
    assert call(_desc(), ws=need - 1) == bgtq.ERR_WORKSPACE
    assert call(_desc(), scale=0.0) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), kv=None) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), kv_dtype=7) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), stride_head=0) == bgtq.ERR_INVALID_ARG
    assert call(_desc(k_norms=None)) == bgtq.ERR_INVALID_ARG


def test_prefill_validation():
    lib = bgtq.lib()
    need = lib.bgtq_prefill_workspace_bytes(2, 1000, 128)
    assert need == lib.bgtq_energy_workspace_bytes(2, 1000, 128)

    def call(desc=None, seq=0, b_min=0, b_max=8, ws=need, n=100, qz=None):
        return lib.bgtq_prefill(ctypes.byref(qz or _quantizer()), ctypes.byref(desc or _desc()), seq, FAKE, FAKE, 0, n,
                                1024 * 128, 128, b_min, b_max, None, FAKE, ws, None)

    assert call(seq=1) == bgtq.ERR_INVALID_ARG                     # batch of one
    assert call(b_min=4) == bgtq.ERR_BUDGET                        # 192 < 64 * 4
    assert call(b_max=2) == bgtq.ERR_BUDGET                        # 192 > 64 * 2
    assert call(b_max=9) == bgtq.ERR_BUDGET
    assert call(n=0) == bgtq.ERR_INVALID_ARG
    assert call(n=257) == bgtq.ERR_CAPACITY                        # capacity 256
    assert call(ws=lib.bgtq_prefill_workspace_bytes(2, 100, 128) - 1) == bgtq.ERR_WORKSPACE
    assert call(qz=bgtq.Quantizer(None, None, None, None, 128, bgtq.ROT_GIVENS, None)) == bgtq.ERR_INVALID_ARG


def test_rotation_kind_validation():
    lib = bgtq.lib()
    need = lib.bgtq_decode_workspace_bytes(1, 16, 2, 128, 256)

    def decode(qz):
        return lib.bgtq_decode_attention(ctypes.byref(qz), ctypes.byref(_desc()), 16, FAKE, 0, None, 1e6, 0.0,
                                         FAKE, None, FAKE, need, None)

    # a valid quantizer gets as far as the softmax-scale check (scale 0 is invalid)
    assert decode(bgtq.Quantizer(None, None, None, None, 128, bgtq.ROT_GIVENS, FAKE)) == bgtq.ERR_INVALID_ARG
    assert b"softmax_scale" in lib.bgtq_last_error()
    assert decode(bgtq.Quantizer(None, None, None, None, 128, bgtq.ROT_GIVENS, None)) == bgtq.ERR_INVALID_ARG
    assert b"givens" in lib.bgtq_last_error()
    assert decode(bgtq.Quantizer(FAKE, FAKE, FAKE, FAKE, 128, 2, FAKE)) == bgtq.ERR_INVALID_ARG
    assert b"rotation kind" in lib.bgtq_last_error()
    assert decode(bgtq.Quantizer(None, FAKE, FAKE, FAKE, 128, bgtq.ROT_DENSE, FAKE)) == bgtq.ERR_INVALID_ARG


def test_window_validation():
    lib = bgtq.lib()
    need = lib.bgtq_decode_workspace_bytes(1, 16, 2, 128, 256)

    def decode(desc):
        return lib.bgtq_decode_attention(ctypes.byref(_quantizer()), ctypes.byref(desc), 16, FAKE, 0, None, 1e6,
                                         0.088, FAKE, None, FAKE, need, None)

    assert decode(_desc(window=4097, k_window=FAKE)) == bgtq.ERR_INVALID_ARG
    assert decode(_desc(window=-1, k_window=FAKE)) == bgtq.ERR_INVALID_ARG
    assert decode(_desc(window=64, k_window=None)) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_quantize_append(ctypes.byref(_quantizer()), ctypes.byref(_desc(window=64, k_window=None)), 0, 1,
                                    FAKE, FAKE, 0, 1, 256, 128, 128, None) == bgtq.ERR_INVALID_ARG
    # a window is attended by the matrix-core decode only (groups of at most 8 query heads)
    assert lib.bgtq_decode_attention(ctypes.byref(_quantizer()), ctypes.byref(_desc(window=64, k_window=FAKE)), 32,
                                     FAKE, 0, None, 1e6, 0.088, FAKE, None, FAKE,
                                     lib.bgtq_decode_workspace_bytes(1, 32, 2, 128, 256), None) == bgtq.ERR_UNSUPPORTED


def test_logit_error_validation():
    lib = bgtq.lib()
    need = lib.bgtq_logit_error_workspace_bytes(2, 16, 1024)
    assert need == 2 * 16 * 4 * 8
    assert lib.bgtq_logit_error_workspace_bytes(0, 16, 1024) == 0

    def call(q=FAKE, keys=FAKE, n_q=16, n_kv=2, d=128, strides=(2 * 1024 * 128, 1024 * 128, 128), cap=1024,
             ws=need, scale=0.088, k_dtype=0, pairing=0, logits=FAKE):
        return lib.bgtq_logit_error(q, 0, None, keys, k_dtype, 2, n_q, n_kv, d, *strides, FAKE, cap, pairing, 1e6,
                                    scale, logits, FAKE, FAKE, ws, None)

    assert call(q=None) == bgtq.ERR_INVALID_ARG
    assert call(keys=None) == bgtq.ERR_INVALID_ARG
    assert call(n_q=15) == bgtq.ERR_INVALID_ARG
    assert call(n_q=34) == bgtq.ERR_UNSUPPORTED
    assert call(d=96, strides=(96, 96, 96)) == bgtq.ERR_UNSUPPORTED
    assert call(ws=need - 1) == bgtq.ERR_WORKSPACE
    assert call(scale=0.0) == bgtq.ERR_INVALID_ARG
    assert call(k_dtype=3) == bgtq.ERR_INVALID_ARG
    assert call(pairing=2) == bgtq.ERR_INVALID_ARG
    assert call(strides=(0, 0, 64)) == bgtq.ERR_INVALID_ARG          # stride_token < head_dim
    assert call(strides=(0, 0, 130)) == bgtq.ERR_INVALID_ARG         # not a multiple of 4
    assert call(cap=1022) == bgtq.ERR_INVALID_ARG
    assert call(keys=FAKE + 4) == bgtq.ERR_INVALID_ARG               # misaligned fp32 keys
    assert call(logits=FAKE + 8) == bgtq.ERR_INVALID_ARG


def test_status_strings():
    lib = bgtq.lib()
    for s in range(7):
        assert lib.bgtq_status_string(s)
    assert lib.bgtq_status_string(99) == b"unknown status"


def test_options_round_trip():
    lib = bgtq.lib()
    old_k, old_w = bgtq.get_option(bgtq.OPT_DECODE_KERNEL), bgtq.get_option(bgtq.OPT_STEP_WAIT_LIMIT)
    try:
        bgtq.set_option(bgtq.OPT_DECODE_KERNEL, 1)
        assert bgtq.get_option(bgtq.OPT_DECODE_KERNEL) == 1
        bgtq.set_option(bgtq.OPT_STEP_WAIT_LIMIT, 0)
        assert bgtq.get_option(bgtq.OPT_STEP_WAIT_LIMIT) == 0
        bgtq.set_option(bgtq.OPT_DECODE_KERNEL, 2)
        assert bgtq.get_option(bgtq.OPT_DECODE_KERNEL) == 2
        assert lib.bgtq_set_option(bgtq.OPT_DECODE_KERNEL, 3) == bgtq.ERR_INVALID_ARG
        assert lib.bgtq_set_option(bgtq.OPT_STEP_WAIT_LIMIT, -1) == bgtq.ERR_INVALID_ARG
        assert lib.bgtq_set_option(7, 0) == bgtq.ERR_INVALID_ARG
        assert lib.bgtq_get_option(7) == -1
    finally:
        bgtq.set_option(bgtq.OPT_DECODE_KERNEL, old_k)
        bgtq.set_option(bgtq.OPT_STEP_WAIT_LIMIT, old_w)


def test_decode_step_noalloc_validation():
    """Host checks of the allocation-free step: a cache whose decode workspace exceeds the scratch
    is refused, and bad arguments are refused before any device is touched."""
    lib = bgtq.lib()

    def call(desc, n_q=16, scale=0.088, kv=FAKE):
        return lib.bgtq_decode_step_noalloc(ctypes.byref(_quantizer()), ctypes.byref(desc), n_q, FAKE, 0, kv, kv, 0,
                                            256, 128, 1e6, scale, FAKE, None, None)

    big = _desc(batch=64, n_kv_heads=8, capacity=1 << 20)
    assert lib.bgtq_decode_workspace_bytes(64, 256, 8, 128, 1 << 20) > bgtq.NOALLOC_SCRATCH_BYTES
    assert call(big, n_q=256) == bgtq.ERR_WORKSPACE
    assert b"scratch" in lib.bgtq_last_error()
    assert lib.bgtq_decode_workspace_bytes(1, 16, 2, 128, 131136) <= bgtq.NOALLOC_SCRATCH_BYTES
    assert call(_desc(), n_q=15) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), n_q=34) == bgtq.ERR_UNSUPPORTED
    assert call(_desc(), scale=0.0) == bgtq.ERR_INVALID_ARG
    assert call(_desc(), kv=None) == bgtq.ERR_INVALID_ARG
    assert call(_desc(k_norms=None)) == bgtq.ERR_INVALID_ARG
    assert lib.bgtq_decode_step_noalloc(ctypes.byref(_quantizer()), None, 16, FAKE, 0, FAKE, FAKE, 0, 256, 128, 1e6,
                                        0.088, FAKE, None, None) == bgtq.ERR_INVALID_ARG


@pytest.mark.parametrize("batch,n_q,n_kv,d,ksum,vb,cap", [
    (1, 8, 1, 128, 192, 3, 5056),      # one KV head: the streamed pass runs 255 splits
    (1, 1, 1, 64, 96, 3, 320),
    (1, 16, 2, 128, 192, 3, 131136),
    (2, 2, 1, 64, 0, 3, 128),
    (16, 28, 4, 128, 192, 2, 65600),
    (1, 32, 8, 128, 128, 2, 32832),
    (3, 12, 3, 256, 384, 4, 640),
    (64, 64, 8, 128, 512, 8, 64),
])
def test_decode_workspace_covers_every_split_count(batch, n_q, n_kv, d, ksum, vb, cap):
    """A workspace of exactly bgtq_decode_workspace_bytes passes the host's own check of the
    partial-result layout for whichever pass serves the cache (the call then stops at the
    missing GPU, never at the workspace)."""
    lib = bgtq.lib()
    need = lib.bgtq_decode_workspace_bytes(batch, n_q, n_kv, d, cap)
    desc = _desc(batch=batch, n_kv_heads=n_kv, head_dim=d, k_width_sum=ksum, v_bits=vb, capacity=cap)
    for opt in (0, 1, 2):
        old = bgtq.get_option(bgtq.OPT_DECODE_KERNEL)
        bgtq.set_option(bgtq.OPT_DECODE_KERNEL, opt)
        try:
            st = lib.bgtq_decode_attention(ctypes.byref(_quantizer(d)), ctypes.byref(desc), n_q, FAKE, 0, None, 1e6,
                                           0.088, FAKE, None, FAKE, need, None)
        finally:
            bgtq.set_option(bgtq.OPT_DECODE_KERNEL, old)
        assert st != bgtq.ERR_WORKSPACE, lib.bgtq_last_error()
        assert st in (bgtq.OK, bgtq.ERR_HIP, bgtq.ERR_UNSUPPORTED)
