"""Decode attention over the packed cache, by its literal definition (oracle, fp64).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the packed-cache
serving path attends over the quantized cache (packed K3V3 at 128K context),
and the quantity the method protects is the RoPE query-key logit.

Definition used here: every cached key and value is dequantized (TQ-MSE
reconstruction, width-0 blocks as zero); the query is rotated by RoPE at its
position; logits are scale * q_rope . k_hat_t over all cached tokens t (no
mask: every cached position precedes the query); the output is the softmax-
weighted sum of the dequantized values.  Grouped-query attention maps query
head h to KV head h // (H_q / H_kv).  Everything is fp64; the softmax subtracts
the maximum before exponentiating.
"""

from __future__ import annotations

import numpy as np

from . import rope


def attend(q_rope, k_hat, v_hat, scale: float):
    """One query head: (out [d], logits [T]) in fp64."""
    s = scale * (np.asarray(k_hat, dtype=np.float64) @ np.asarray(q_rope, dtype=np.float64))
    if s.shape[0] == 0:
        return np.zeros(v_hat.shape[-1]), s
    w = np.exp(s - np.max(s))
    p = w / np.sum(w)
    return p @ np.asarray(v_hat, dtype=np.float64), s


def decode_head_group(q, pos, base, k_hat, v_hat, scale=None, pairing=rope.HALF):
    """Query heads q [G, d] (pre-RoPE) sharing one KV head -> (out [G, d], logits [G, T])."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qr = rope.apply(q, pos, base, pairing) if base > 0 else q
    outs, logits = [], []
    for h in range(q.shape[0]):
        o, s = attend(qr[h], k_hat, v_hat, scale)
        outs.append(o)
        logits.append(s)
    return np.stack(outs), np.stack(logits)
