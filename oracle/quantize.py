"""TurboQuant-MSE quantization of keys (per width group) and values (oracle).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: keys are
quantized with TQ-MSE at the per-block widths chosen by the allocator; K and V
budgets are matched, values at a uniform width (K3V3, K2V2, K3V2).

Reading of TQ-MSE for one vector x in R^m at b bits (from the TurboQuant paper,
outside the pages): store the norm n = |x|; rotate with a fixed random
orthogonal m x m matrix Pi; scale so that the coordinates are close to
N(0, 1): z = (Pi x / n) * sqrt(m); code every coordinate with the b-bit
Lloyd-Max quantizer of N(0, 1).  Reconstruction is n * Pi^T (C_b[code] / sqrt(m)),
with C_b the fp16-rounded reconstruction levels and n the stored fp16 norm.
No residual (QJL) stage, no renormalisation.

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


def tq_mse(x, rot, bits: int):
    """Codes [T, m] (int64) and fp16 norms [T] of rows x [T, m] (fp32) with rotation rot [m, m]."""
    x = np.asarray(x, dtype=np.float32)
    rot = np.asarray(rot, dtype=np.float32)
    t_len, m = x.shape
    ss = np.zeros(t_len, dtype=np.float32)
    for i in range(m):
        ss = ss + x[:, i] * x[:, i]
    nrm = np.sqrt(ss)
    y = np.zeros((t_len, m), dtype=np.float32)
    for k in range(m):                                   # ascending k for every output i
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


def bank_matrix(bank, m: int) -> np.ndarray:
    o = bank_offset(m)
    return np.asarray(bank, dtype=np.float32)[o:o + m * m].reshape(m, m)


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


def quantize_values(v, rot_v, bits: int):
    """Values v [T, d] -> (codes [T, d] in rotated coordinate order, norms [T] fp16)."""
    return tq_mse(v, rot_v, bits)


def dequantize_keys(codes, norms, lay: Layout, bank) -> np.ndarray:
    """fp64 reconstruction [T, d] in original coordinate order; width-0 blocks are 0."""
    codes = np.asarray(codes)
    t_len = codes.shape[0]
    out = np.zeros((t_len, lay.d), dtype=np.float64)
    for g, grp in enumerate(lay.groups):
        cen = codebook.levels16(grp.width)
        rot = bank_matrix(bank, grp.m).astype(np.float64)
        yhat = cen[codes[:, grp.first:grp.first + grp.m]] / np.sqrt(grp.m)
        xg = (yhat @ rot) * norms[:, g].astype(np.float64)[:, None]   # rows: Pi^T yhat
        out[:, lay.perm[grp.first:grp.first + grp.m]] = xg
    return out


def dequantize_values(codes, norms, rot_v, bits: int) -> np.ndarray:
    d = rot_v.shape[0]
    cen = codebook.levels16(bits)
    yhat = cen[np.asarray(codes)] / np.sqrt(d)
    return (yhat @ np.asarray(rot_v, dtype=np.float64)) * np.asarray(norms, dtype=np.float64)[:, None]
