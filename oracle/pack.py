"""Byte layout of the packed K/V cache (oracle).

The pages report a packed-cache serving path (packed K3V3, 3.24x KV
compression; RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract,
serving-path sentences) but give no layout.  This is the layout of this
implementation, stated so that every packed byte can be checked:

One (sequence, KV head) region of capacity C tokens (C a multiple of 64) is
split into C/64 tiles of 64 token slots; slot s of tile tau holds token
t = 64*tau + s.

* K codes: each token's record is its codes in storage order, LSB first
  (record bit i is bit i%8 of record byte i//8; the code at storage position p
  occupies bits [offset[p], offset[p] + width[p])), zero-padded to `chunks`
  16-byte chunks.  Chunk c of slot s of tile tau is stored at byte
  ((tau*chunks + c)*64 + s)*16, so the 64 slots' copies of one chunk are 1 KiB
  of contiguous memory.
* K norms: fp16, group g of slot s of tile tau at element (tau*8 + g)*64 + s
  (room for the at most 8 width groups of widths 1..8).
* V codes: coordinate-major per tile: rotated coordinate r of tile tau owns a
  segment of 64*b_v bits (8*b_v bytes) at byte (tau*d + r)*8*b_v, and slot s
  holds its code at segment bits [s*b_v, (s+1)*b_v), LSB first.
* V norms: fp16, slot s of tile tau at element tau*64 + s.

Unused slots and padding bits are zero.
"""

from __future__ import annotations

import numpy as np

from .layout import Layout

TILE = 64
MAX_GROUPS = 8


def _bits_le(codes, widths, offsets, total_bits) -> np.ndarray:
    """Rows of LSB-first bits: out[t, offsets[p] + i] = bit i of codes[t, p]."""
    codes = np.asarray(codes, dtype=np.int64)
    out = np.zeros((codes.shape[0], total_bits), dtype=np.uint8)
    for p in range(codes.shape[1]):
        for i in range(int(widths[p])):
            out[:, int(offsets[p]) + i] = (codes[:, p] >> i) & 1
    return out


def k_record_bytes(codes, lay: Layout) -> np.ndarray:
    """[T, 16*chunks] record bytes of every token."""
    bits = _bits_le(codes, lay.width, lay.offset, lay.chunks * 128)
    return np.packbits(bits, axis=1, bitorder="little")


def region_sizes(d: int, chunks: int, v_bits: int, capacity: int) -> dict:
    tiles = capacity // TILE
    return {
        "k_codes": tiles * chunks * TILE * 16,
        "k_norms": tiles * MAX_GROUPS * TILE,          # fp16 elements
        "v_codes": tiles * d * 8 * v_bits,
        "v_norms": tiles * TILE,                       # fp16 elements
    }


def pack_region(k_codes, k_norms, v_codes, v_norms, lay: Layout, v_bits: int, capacity: int) -> dict:
    """Cache region of one (sequence, KV head) holding tokens 0..T-1."""
    if capacity % TILE:
        raise ValueError("capacity must be a multiple of 64")
    t_len = np.asarray(k_codes).shape[0]
    if t_len > capacity:
        raise ValueError("more tokens than capacity")
    d = lay.d
    tiles = capacity // TILE
    t = np.arange(t_len)
    tau, slot = t // TILE, t % TILE

    kc = np.zeros((tiles, lay.chunks, TILE, 16), dtype=np.uint8)
    rec = k_record_bytes(k_codes, lay)
    for c in range(lay.chunks):
        kc[tau, c, slot, :] = rec[:, 16 * c:16 * (c + 1)]

    kn = np.zeros((tiles, MAX_GROUPS, TILE), dtype=np.float16)
    for g in range(len(lay.groups)):
        kn[tau, g, slot] = np.asarray(k_norms)[:, g]

    vbits = np.zeros((tiles, d, TILE * v_bits), dtype=np.uint8)
    vcodes = np.asarray(v_codes, dtype=np.int64)
    for i in range(v_bits):
        vbits[tau[:, None], np.arange(d)[None, :], (slot * v_bits + i)[:, None]] = (vcodes >> i) & 1
    vc = np.packbits(vbits, axis=2, bitorder="little")   # [tiles, d, 8*v_bits]

    vn = np.zeros((tiles, TILE), dtype=np.float16)
    vn[tau, slot] = np.asarray(v_norms)

    return {"k_codes": kc.reshape(-1), "k_norms": kn.reshape(-1),
            "v_codes": vc.reshape(-1), "v_norms": vn.reshape(-1)}


def unpack_region(region: dict, lay: Layout, v_bits: int, t_len: int):
    """Inverse of pack_region for tokens 0..t_len-1: (k_codes, k_norms, v_codes, v_norms)."""
    d = lay.d
    kc = np.asarray(region["k_codes"], dtype=np.uint8)
    tiles = kc.shape[0] // max(1, lay.chunks * TILE * 16) if lay.chunks else 0
    t = np.arange(t_len)
    tau, slot = t // TILE, t % TILE
    if lay.chunks:
        kc = kc.reshape(tiles, lay.chunks, TILE, 16)
        rec = np.concatenate([kc[tau, c, slot, :] for c in range(lay.chunks)], axis=1)
        bits = np.unpackbits(rec, axis=1, bitorder="little").astype(np.int64)
    k_codes = np.zeros((t_len, lay.d_eff), dtype=np.int64)
    for p in range(lay.d_eff):
        for i in range(int(lay.width[p])):
            k_codes[:, p] |= bits[:, int(lay.offset[p]) + i] << i
    kn = np.asarray(region["k_norms"], dtype=np.float16).reshape(-1, MAX_GROUPS, TILE)
    k_norms = np.stack([kn[tau, g, slot] for g in range(len(lay.groups))], axis=1) \
        if lay.groups else np.zeros((t_len, 0), dtype=np.float16)
    vc = np.asarray(region["v_codes"], dtype=np.uint8).reshape(-1, d, 8 * v_bits)
    vbits = np.unpackbits(vc, axis=2, bitorder="little").astype(np.int64)
    v_codes = np.zeros((t_len, d), dtype=np.int64)
    for i in range(v_bits):
        v_codes |= vbits[tau[:, None], np.arange(d)[None, :], (slot * v_bits + i)[:, None]] << i
    vn = np.asarray(region["v_norms"], dtype=np.float16).reshape(-1, TILE)
    return k_codes, k_norms, v_codes, vn[tau, slot]
