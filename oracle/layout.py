"""Width groups and the K record bit layout derived from an allocation (oracle).

Reading ("width-group TQ-MSE"; the pages only say that Block-GTQ is built on
TQ-MSE and gives each RoPE block its own integer width): the blocks that
received the same width b >= 1 form one group.  The group's coordinates, taken
block by block in ascending block index with each block's first coordinate
before its second, form a sub-vector of size m = 2 * (number of blocks) that is
coded as one TQ-MSE vector at b bits per coordinate, with its own norm and its
own m x m rotation.  Rotations never mix blocks of different widths, so block j
is coded at exactly b_j bits per coordinate.  Blocks of width 0 are dropped
(reconstructed as zero).

Groups are ordered by descending width.  Concatenating the groups' coordinates
in that order gives the *storage order*: storage position p holds original
coordinate perm[p], coded with width[p] bits at bit offset offset[p] of the
token's K record.  The record holds sum_j 2*b_j = 2B code bits and is padded to
a whole number of 16-byte chunks.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .rope import block_coords, HALF


@dataclass(frozen=True)
class Group:
    width: int          # bits per coordinate
    blocks: tuple       # RoPE block indices, ascending
    first: int          # first storage position
    m: int              # number of coordinates = 2 * len(blocks)
    bit_offset: int     # bit offset of the group's first code in the record


@dataclass(frozen=True)
class Layout:
    d: int
    groups: tuple
    perm: np.ndarray        # storage position -> original coordinate
    width: np.ndarray       # storage position -> bits
    offset: np.ndarray      # storage position -> bit offset in the record
    code_bits: int          # 2B
    chunks: int             # 16-byte chunks per record

    @property
    def d_eff(self) -> int:
        return int(self.perm.shape[0])


def build(widths, pairing: int = HALF) -> Layout:
    widths = [int(w) for w in widths]
    n = len(widths)
    d = 2 * n
    a, b = block_coords(d, pairing)
    groups, perm, wid, off = [], [], [], []
    pos, bit = 0, 0
    for w in range(8, 0, -1):
        blocks = tuple(j for j in range(n) if widths[j] == w)
        if not blocks:
            continue
        groups.append(Group(w, blocks, pos, 2 * len(blocks), bit))
        for j in blocks:
            for c in (a[j], b[j]):
                perm.append(int(c))
                wid.append(w)
                off.append(bit)
                bit += w
                pos += 1
    code_bits = bit
    return Layout(d=d, groups=tuple(groups),
                  perm=np.array(perm, dtype=np.int64),
                  width=np.array(wid, dtype=np.int64),
                  offset=np.array(off, dtype=np.int64),
                  code_bits=code_bits,
                  chunks=-(-code_bits // 128))
