"""fp16 recent-key window beside the packed cache (oracle, fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the AIME result is
stated to hold without an fp16 recent-key buffer, which implies the serving path can
keep one: the newest keys held in fp16 instead of (or beside) their quantized form.

Readings (the pages name the buffer and nothing more):

* The window holds the keys of the newest W tokens of a sequence, t in
  [max(0, T - W), T) for T cached tokens; W = 0 means no window.
* A key in the window is its post-RoPE value rounded to fp16 (nearest-even),
  saturated at +-65504 (the cache's fp16 norms saturate the same way).
* Attention uses that fp16 key in place of the key's TQ-MSE reconstruction; values
  stay quantized (the buffer is named for keys only).  Softmax runs over all T
  tokens at once, so the window changes logits, not the attention structure.
"""

from __future__ import annotations

import numpy as np

from . import decode, rope

FP16_MAX = 65504.0


def fp16_keys(keys) -> np.ndarray:
    """Keys rounded to fp16 (nearest-even) after saturation at +-65504, as fp64 values."""
    k = np.clip(np.asarray(keys, dtype=np.float64), -FP16_MAX, FP16_MAX)
    return k.astype(np.float16).astype(np.float64)


def window_range(t_len: int, window: int) -> tuple[int, int]:
    """Tokens [lo, hi) whose keys the window holds."""
    if window <= 0:
        return t_len, t_len
    return max(0, t_len - window), t_len


def effective_keys(k_hat, keys, window: int) -> np.ndarray:
    """Keys attention uses: k_hat [T, d] with the window's rows replaced by fp16 keys."""
    k_eff = np.array(k_hat, dtype=np.float64, copy=True)
    lo, hi = window_range(k_eff.shape[0], window)
    k_eff[lo:hi] = fp16_keys(np.asarray(keys)[lo:hi])
    return k_eff


def decode_head_group(q, pos, base, k_hat, keys, v_hat, window: int, scale=None, pairing=rope.HALF):
    """Query heads q [G, d] over one KV head's cache with a window -> (out [G, d], logits [G, T])."""
    return decode.decode_head_group(q, pos, base, effective_keys(k_hat, keys, window), v_hat, scale=scale,
                                    pairing=pairing)


def ring_slots(t_len: int, window: int) -> dict:
    """Slot of each windowed token in a ring of `window` slots: token t at t mod window."""
    lo, hi = window_range(t_len, window)
    return {t: t % window for t in range(lo, hi)}
