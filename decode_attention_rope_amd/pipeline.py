"""Prefill and decode steps of the library.

Prefill of one sequence (per layer): block energy of its keys, greedy widths
under the K budget, then quantize-and-append of the whole prompt, in one
bgtq_prefill call.  A decode step: append the new token's key and value, then
attend (the query's own token is the newest cached one), in one
bgtq_decode_step call.  Every step runs in the HIP library.
"""

from __future__ import annotations

import torch

from . import bgtq


def prefill(quantizer, cache: bgtq.PackedCache, keys: torch.Tensor, values: torch.Tensor, seq: int,
            b_min: int = 0, b_max: int = 8) -> None:
    """keys, values [n_kv_heads, T, head_dim] of sequence `seq` (post-RoPE keys)."""
    bgtq.bgtq_prefill(quantizer, cache, keys, values, seq, b_min, b_max)


def decode_step(quantizer, cache: bgtq.PackedCache, k_new: torch.Tensor, v_new: torch.Tensor,
                q: torch.Tensor, rope_theta: float, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """k_new, v_new [batch, n_kv_heads, 1, head_dim]; q [batch, n_q_heads, head_dim] (pre-RoPE).
    One bgtq_decode_step call: the same result as appending, then attending."""
    return bgtq.bgtq_decode_step(quantizer, cache, q, k_new, v_new, rope_theta, out=out, workspace=workspace)
