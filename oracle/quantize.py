"""TurboQuant-MSE quantization of keys (per width group) and values (oracle).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: keys are
quantized with TQ-MSE at the per-block widths chosen by the allocator; K and V
budgets are matched, values at a uniform width (K3V3, K2V2, K3V2).

Reading of TQ-MSE for one vector x in R^m at b bits (from the TurboQuant paper,
outside the pages): store the norm n = |x|; rotate with a fixed random
orthogonal m x m matrix Pi; scale so that the coordinates are close to
N(0, 1): z = (Pi x / n) * sqrt(m); code every coordinate with the b-bit
Lloyd-Max quantizer of N(0, 1).  Reconstruction is n * Pi^T (C_b[code] / sqrt(m)),
with C_b the fp32 Lloyd-Max centroids and n the stored fp16 norm.
No residual (QJL) stage, no renormalisation.

Structured rotations (the second rotation kind; the pages fix no rotation type): Pi may
instead be a product of Givens layers S_m = G_L ... G_1.  Layer G_l rotates each pair
(a, b) of a perfect matching of the m coordinates by its angle: y_a = c x_a - s x_b,
y_b = s x_a + c x_b, with fp32 cos and sin drawn with the input.  Forward, every product
and every difference or sum is rounded to fp32 (no fused multiply-add), layer by layer.
The reconstruction uses the transpose S_m^T (layers in reverse order, each as
[[c, s], [-s, c]]), in fp64, exactly as the dense path uses Pi^T.

Bit-exact arithmetic (so that a GPU kernel can reproduce every code and norm):

* x is taken in fp32 (bf16 inputs widen exactly);
* ss = fp32 sequential sum over the sub-vector of x_i * x_i, each product and
  each add rounded to fp32 (no fused multiply-add); n = sqrt(ss) rounded to fp32;
* y_i = fp32 sequential sum over k of Pi[i, k] * x_k (ascending k, no FMA);
* z_i = (y_i / n) * S_m with S_m = fl32(sqrt(m)), every step rounded to fp32;
* code_i = number of fp32 thresholds T_b[k] with z_i > T_b[k];
* the stored norm is n rounded to fp16 (nearest-even), saturated at 65504;
* a zero vector (n == 0) gets all-zero codes and stored norm +0.
"""

from __future__ import annotations

import numpy as np

from . import codebook
from .layout import Layout

FP16_MAX = np.float32(65504.0)


class Givens:
    """Givens-layer rotations for every even size, read from the packed array the input
    generator draws: header row m/2 - 1 = (first record row, layer count), then records
    (a | b << 16, fp32 bits of cos, fp32 bits of sin, 0)."""

    def __init__(self, records):
        self.rec = np.asarray(records, dtype=np.uint32)

    def layers(self, m: int):
        """[(a, b, c, s)] per layer for size m; a, b index the m coordinates, c, s fp32."""
        first, n_layers = int(self.rec[m // 2 - 1, 0]), int(self.rec[m // 2 - 1, 1])
        out = []
        for l in range(n_layers):
            r = self.rec[first + l * (m // 2): first + (l + 1) * (m // 2)]
            out.append(((r[:, 0] & 0xFFFF).astype(np.int64), (r[:, 0] >> 16).astype(np.int64),
                        r[:, 1].view(np.float32), r[:, 2].view(np.float32)))
        return out

    def matrix(self, m: int) -> np.ndarray:
        """S_m as a dense fp64 matrix (product of the layers with the fp32 cos and sin)."""
        return givens_forward64(np.eye(m), self.layers(m)).T


def givens_forward32(x, layers) -> np.ndarray:
    """y = S x for rows x [T, m] in fp32, layer by layer, every product and sum rounded."""
    y = np.array(x, dtype=np.float32, copy=True)
    for a, b, c, s in layers:
        xa, xb = y[:, a].copy(), y[:, b].copy()
        y[:, a] = (c * xa) - (s * xb)
        y[:, b] = (s * xa) + (c * xb)
    return y


def givens_forward64(x, layers) -> np.ndarray:
    """y = S x for rows x [T, m] in fp64 (the cos and sin as stored)."""
    y = np.array(x, dtype=np.float64, copy=True)
    for a, b, c, s in layers:
        c64, s64 = c.astype(np.float64), s.astype(np.float64)
        xa, xb = y[:, a].copy(), y[:, b].copy()
        y[:, a] = c64 * xa - s64 * xb
        y[:, b] = s64 * xa + c64 * xb
    return y


def givens_transpose64(y, layers) -> np.ndarray:
    """x = S^T y for rows y [T, m] in fp64: layers in reverse order, each transposed."""
    x = np.array(y, dtype=np.float64, copy=True)
    for a, b, c, s in reversed(layers):
        c64, s64 = c.astype(np.float64), s.astype(np.float64)
        ya, yb = x[:, a].copy(), x[:, b].copy()
        x[:, a] = c64 * ya + s64 * yb
        x[:, b] = -s64 * ya + c64 * yb
    return x


def tq_mse(x, rot, bits: int):
    """Codes [T, m] (int64) and fp16 norms [T] of rows x [T, m] (fp32) with rotation rot: a
    dense [m, m] matrix or a list of Givens layers."""
    x = np.asarray(x, dtype=np.float32)
    t_len, m = x.shape
    ss = np.zeros(t_len, dtype=np.float32)
    for i in range(m):
        ss = ss + x[:, i] * x[:, i]
    nrm = np.sqrt(ss)
    if isinstance(rot, list):
        y = givens_forward32(x, rot)
    else:
        rot = np.asarray(rot, dtype=np.float32)
        y = np.zeros((t_len, m), dtype=np.float32)
        for k in range(m):                               # ascending k for every output i
            y = y + rot[:, k][None, :] * x[:, k][:, None]
    safe = np.where(nrm == 0, np.float32(1.0), nrm)
    z = (y / safe[:, None]) * np.float32(np.sqrt(np.float32(m)))
    thr = codebook.thresholds32(bits)
    codes = np.zeros((t_len, m), dtype=np.int64)
    for k in range(thr.shape[0]):                        # count thresholds strictly below z
        codes += (z > thr[k]).astype(np.int64)
    codes[nrm == 0] = 0
    stored = np.minimum(nrm, FP16_MAX).astype(np.float16)
    return codes, stored


def bank_offset(m: int) -> int:
    """Offset (in floats) of the m x m matrix in the concatenated bank m = 2, 4, ..., d."""
    return sum(k * k for k in range(2, m, 2))


def bank_matrix(bank, m: int):
    """The size-m rotation of a bank: dense fp32 [m, m], or the Givens layers of a Givens bank."""
    if isinstance(bank, Givens):
        return bank.layers(m)
    o = bank_offset(m)
    return np.asarray(bank, dtype=np.float32)[o:o + m * m].reshape(m, m)


def _unrotate(yhat, rot) -> np.ndarray:
    """Rows Pi^T yhat in fp64 for a dense rotation or Givens layers."""
    if isinstance(rot, list):
        return givens_transpose64(yhat, rot)
    return yhat @ np.asarray(rot, dtype=np.float64)


def quantize_keys(k, lay: Layout, bank):
    """Post-RoPE keys k [T, d] -> (codes [T, d_eff] in storage order, norms [T, groups] fp16)."""
    k = np.asarray(k, dtype=np.float32)
    t_len = k.shape[0]
    codes = np.zeros((t_len, lay.d_eff), dtype=np.int64)
    norms = np.zeros((t_len, len(lay.groups)), dtype=np.float16)
    for g, grp in enumerate(lay.groups):
        cols = lay.perm[grp.first:grp.first + grp.m]
        c, n = tq_mse(k[:, cols], bank_matrix(bank, grp.m), grp.width)
        codes[:, grp.first:grp.first + grp.m] = c
        norms[:, g] = n
    return codes, norms


def value_rotation(rot_v, d: int):
    """The value rotation: a dense [d, d] matrix, or the size-d layers of a Givens bank."""
    return rot_v.layers(d) if isinstance(rot_v, Givens) else rot_v


def quantize_values(v, rot_v, bits: int):
    """Values v [T, d] -> (codes [T, d] in rotated coordinate order, norms [T] fp16)."""
    return tq_mse(v, value_rotation(rot_v, np.asarray(v).shape[-1]), bits)


def _levels(bits: int, levels: str) -> np.ndarray:
    """Reconstruction levels as fp64 values: "fp32" = the fp32 Lloyd-Max centroids (the
    reconstruction the method defines), "fp16" = those rounded once more to fp16."""
    if levels == "fp16":
        return codebook.levels16(bits)
    if levels == "fp32":
        return codebook.centroids32(bits).astype(np.float64)
    raise ValueError(f"levels must be 'fp16' or 'fp32', not {levels!r}")


def dequantize_keys(codes, norms, lay: Layout, bank, levels: str = "fp32") -> np.ndarray:
    """fp64 reconstruction [T, d] in original coordinate order; width-0 blocks are 0."""
    codes = np.asarray(codes)
    t_len = codes.shape[0]
    out = np.zeros((t_len, lay.d), dtype=np.float64)
    for g, grp in enumerate(lay.groups):
        cen = _levels(grp.width, levels)
        yhat = cen[codes[:, grp.first:grp.first + grp.m]] / np.sqrt(grp.m)
        xg = _unrotate(yhat, bank_matrix(bank, grp.m)) * norms[:, g].astype(np.float64)[:, None]
        out[:, lay.perm[grp.first:grp.first + grp.m]] = xg
    return out


def dequantize_values(codes, norms, rot_v, bits: int, levels: str = "fp32") -> np.ndarray:
    d = np.asarray(codes).shape[-1]
    cen = _levels(bits, levels)
    yhat = cen[np.asarray(codes)] / np.sqrt(d)
    return _unrotate(yhat, value_rotation(rot_v, d)) * np.asarray(norms, dtype=np.float64)[:, None]
