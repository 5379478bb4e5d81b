"""Key-only RoPE logit error of Block-GTQ against uniform TQ-MSE (oracle, fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring): the tests, the smoke check
and the CPU baseline may call this; the HIP library never does.

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: under matched K/V
bit budgets Block-GTQ keeps the RoPE query-key logits closer to their exact
values than uniform TQ-MSE; the measure is the per-layer mean absolute logit
error with only the keys quantized, at 2 and 3 bits per coordinate.

Readings (the pages give the measure, not its formula):

* Exact logit of query head h and cached token t: e_t = scale * RoPE(q_h, pos) . k_t
  with k_t the unquantized post-RoPE key, scale = 1/sqrt(d) unless given and pos
  the query position (the newest cached token unless given).
* Quantized logit: the same with k_t replaced by its TQ-MSE reconstruction k_hat_t
  (width-0 blocks reconstruct as zero).  Values play no part ("K-only").
* Error of one (sequence, layer, query head): mean over the cached tokens of
  |quantized - exact|; the per-layer figure is the mean over the layer's heads
  and sequences, weighted by token count.
* Uniform TQ-MSE at b bits per coordinate = every block at width b, i.e. one
  width group of all d coordinates with the d x d rotation.  Block-GTQ at b bits
  per coordinate = the greedy widths of the layer-and-head energies under the
  budget b * d/2 (the same budget).

Pins: the logit assembly against the relative-position form of RoPE, a
perturbed-key closed form, flat energies (where Block-GTQ reduces to uniform),
the Gaussian error model of a rotated scalar quantizer, and the direction the
abstract reports on skewed energy profiles.  The magnitude the abstract quotes
(32-80 % lower error on trained models) is not pinned: it needs real models.
"""

from __future__ import annotations

import numpy as np

from . import allocate, energy, layout, quantize, rope


def exact_logits(q, pos, base: float, keys, scale=None, pairing: int = rope.HALF) -> np.ndarray:
    """q [H, d] pre-RoPE query heads, keys [T, d] post-RoPE -> logits [H, T] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qr = rope.apply(q, pos, base, pairing) if base > 0 else q
    return scale * (qr @ np.asarray(keys, dtype=np.float64).T)


def uniform_widths(d: int, bits: int) -> np.ndarray:
    """Uniform TQ-MSE at `bits` bits per coordinate: every RoPE block at that width."""
    return np.full(d // 2, bits, dtype=np.int64)


def block_gtq_widths(keys, bits: int, pairing: int = rope.HALF) -> np.ndarray:
    """Greedy widths of one head's keys [T, d] at the matched budget bits * d/2."""
    k = np.asarray(keys)
    return allocate.greedy(energy.block_energy(k, pairing), bits * (k.shape[-1] // 2))


def reconstruct(keys, widths, bank, pairing: int = rope.HALF) -> np.ndarray:
    """TQ-MSE round trip of keys [T, d] at the given block widths -> k_hat [T, d] fp64."""
    lay = layout.build(widths, pairing)
    codes, norms = quantize.quantize_keys(keys, lay, bank)
    return quantize.dequantize_keys(codes, norms, lay, bank)


def logit_mae(q, pos, base: float, keys, k_hat, scale=None, pairing: int = rope.HALF) -> np.ndarray:
    """Mean over tokens of |quantized - exact| logit, per query head -> [H] (0 for no tokens)."""
    keys = np.asarray(keys)
    if keys.shape[0] == 0:
        return np.zeros(np.asarray(q).shape[0])
    ex = exact_logits(q, pos, base, keys, scale, pairing)
    qu = exact_logits(q, pos, base, k_hat, scale, pairing)
    return np.mean(np.abs(qu - ex), axis=-1)


def k_only_mae(q, pos, base: float, keys, bits: int, bank, method: str, scale=None,
               pairing: int = rope.HALF) -> np.ndarray:
    """Per-head key-only logit MAE of one KV head's query group q [G, d] over keys [T, d].

    method: "uniform" (uniform TQ-MSE) or "block_gtq" (greedy widths, same budget)."""
    d = np.asarray(keys).shape[-1]
    if method == "uniform":
        w = uniform_widths(d, bits)
    elif method == "block_gtq":
        w = block_gtq_widths(keys, bits, pairing)
    else:
        raise ValueError(method)
    return logit_mae(q, pos, base, keys, reconstruct(keys, w, bank, pairing), scale, pairing)
