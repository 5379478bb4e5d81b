"""Per-block energy score that needs no labels (oracle).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the allocator
scores every RoPE frequency block separately per layer and per KV head, using
no labels, and blocks with more energy are the ones that matter most for the
logit error.

Reading (no formula on the pages): the score of block j is the mean over the
sequence's cached keys of the squared norm of the block's two coordinates,

    E_j = (1/T) * sum_t (k[t, a_j]^2 + k[t, b_j]^2).

It uses keys only, so no labels or queries are needed, and RoPE leaves it
unchanged because RoPE rotates each block rigidly.

Arithmetic (so that a GPU reduction can reproduce it bit for bit): inputs are
widened to fp64 (exact for fp32 and bf16); each term k0*k0 + k1*k1 is one fp64
product pair and one fp64 add; terms are summed in ascending t within chunks of
CHUNK tokens, the chunk sums are added in ascending chunk order, and the total
is divided by T.
"""

from __future__ import annotations

import numpy as np

from .rope import block_coords, HALF

CHUNK = 256


def block_energy(keys, pairing: int = HALF) -> np.ndarray:
    """keys [..., T, d] (fp32 or exactly-representable values) -> E [..., d/2] fp64."""
    k = np.asarray(keys)
    t_len, d = k.shape[-2], k.shape[-1]
    if t_len == 0:
        raise ValueError("energy of an empty key set is undefined")
    a, b = block_coords(d, pairing)
    k0 = k[..., a].astype(np.float64)
    k1 = k[..., b].astype(np.float64)
    e = k0 * k0 + k1 * k1                                   # [..., T, n]
    n_chunks = -(-t_len // CHUNK)
    pad = n_chunks * CHUNK - t_len
    if pad:
        # adding +0.0 to a non-negative fp64 sum leaves it unchanged
        e = np.concatenate([e, np.zeros(e.shape[:-2] + (pad, e.shape[-1]))], axis=-2)
    e = e.reshape(e.shape[:-2] + (n_chunks, CHUNK, e.shape[-1]))
    chunk_sum = np.zeros(e.shape[:-3] + (n_chunks, e.shape[-1]))
    for t in range(CHUNK):                                  # ascending t inside a chunk
        chunk_sum = chunk_sum + e[..., :, t, :]
    total = np.zeros(e.shape[:-3] + (e.shape[-1],))
    for c in range(n_chunks):                               # ascending chunk order
        total = total + chunk_sum[..., c, :]
    return total / float(t_len)
