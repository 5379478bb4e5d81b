"""Seeded synthetic inputs for the packed-cache decode path.

This module only draws random inputs; it holds none of the method's arithmetic
(no energy, allocation, quantization or attention).  Both the HIP path and the
CPU oracle are fed from here, so they always see the same bytes.

Every stream is ``numpy.random.default_rng(SeedSequence(seed, spawn_key=...))``
with a spawn key (workload id, sequence, layer, head, stream, block), so any
slice of any tensor can be regenerated on its own.  Keys are drawn pre-RoPE in
fp64 as N(0, sigma_j^2) per coordinate of RoPE block j, rotated to their cache
positions the way a model applies RoPE before caching (angle pos * base^(-2j/d)
in fp64, half pairing), then rounded to the workload's key dtype.  Values are
N(0, 1).  Queries are pre-RoPE with their KV head's sigma profile.

The random rotations TQ-MSE draws (one Haar matrix per even size m = 2..d for
the key width groups, one d x d matrix for values) are generated here too: a
random draw of the method is an input, not part of its arithmetic.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GEN_BLOCK = 8192          # tokens per independently seeded key/value block

_STREAMS = {"profile": 1, "k": 2, "v": 3, "q": 4, "len": 5, "rot": 6, "rotv": 7, "outl": 8, "givens": 9}


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                  # workload id used in spawn keys
    d: int
    h_q: int
    h_kv: int
    theta: float
    layers: int
    seq_lens: tuple           # cached tokens per sequence before decoding
    k_bits: int               # K bits per coordinate (budget B = k_bits * d/2)
    v_bits: int
    key_dtype: str            # "f32" or "bf16"
    profile: str              # "decay", "loguniform", "decay_jitter"
    outlier_blocks: int = 0
    elem_outlier_p: float = 0.0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def n(self) -> int:
        return self.d // 2

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def budget(self) -> int:
        return self.k_bits * self.n


def _rng(wl: Workload, *key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(wl.seed, spawn_key=(wl.wid,) + tuple(int(k) for k in key)))


# ---------------------------------------------------------------- workloads

TINY = Workload("tiny_d64_T256_K3V3", 1, d=64, h_q=1, h_kv=1, theta=1e4, layers=1, seq_lens=(256,),
                k_bits=3, v_bits=3, key_dtype="f32", profile="decay", outlier_blocks=2,
                note="1 layer, 1 KV head, 1 query head, head_dim 64, 256 cached tokens")
LLAMA8B_LAYER = Workload("llama8b_layer_32k_K2V2", 2, d=128, h_q=32, h_kv=8, theta=5e5, layers=1,
                         seq_lens=(32768,), k_bits=2, v_bits=2, key_dtype="bf16", profile="loguniform",
                         elem_outlier_p=0.01,
                         note="Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, 32K cached tokens, bf16 keys")
QWEN3B_128K = Workload("qwen3b_36L_128k_K3V3", 3, d=128, h_q=16, h_kv=2, theta=1e6, layers=36,
                       seq_lens=(131072,), k_bits=3, v_bits=3, key_dtype="f32", profile="decay_jitter",
                       outlier_blocks=2,
                       note="Qwen2.5-3B-shaped decode: 16 q / 2 kv heads, 36 layers, 128K context")
QWEN3B_512K = Workload("qwen3b_36L_512k_K3V3", 4, d=128, h_q=16, h_kv=2, theta=1e6, layers=36,
                       seq_lens=(524288,), k_bits=3, v_bits=3, key_dtype="f32", profile="decay_jitter",
                       outlier_blocks=2,
                       note="Qwen2.5-3B shape at 512K context")


def qwen7b_ragged(seed: int = 0) -> Workload:
    """7B-Qwen-shaped ragged batch: 16 sequences with lengths uniform on [8192, 65536]."""
    proto = Workload("qwen7b_28L_ragged16_K3V2", 5, d=128, h_q=28, h_kv=4, theta=1e6, layers=28,
                     seq_lens=(), k_bits=3, v_bits=2, key_dtype="f32", profile="decay", outlier_blocks=2,
                     seed=seed)
    lens = _rng(proto, 0, 0, 0, _STREAMS["len"]).integers(8192, 65536, size=16, endpoint=True)
    return Workload(proto.name, proto.wid, proto.d, proto.h_q, proto.h_kv, proto.theta, proto.layers,
                    tuple(int(x) for x in lens), proto.k_bits, proto.v_bits, proto.key_dtype,
                    proto.profile, proto.outlier_blocks, seed=seed,
                    note="7B-Qwen-shaped batch of 16 ragged sequences, 28 q / 4 kv heads")


QWEN7B_RAGGED = qwen7b_ragged()

def diagnostic_panel(tokens: int = 4096, layers: int = 4) -> list:
    """Synthetic stand-ins for a panel of models in the key-only logit-error diagnostic: five
    head shapes (head_dim 64/128/256, group sizes 1 to 8) and the three energy profiles, one
    sequence of `tokens` cached tokens, `layers` layers each (k_bits is overridden per run)."""
    def w(name, wid, d, h_q, h_kv, theta, profile, key_dtype="f32", outliers=2, elem_p=0.0):
        return Workload(name, wid, d=d, h_q=h_q, h_kv=h_kv, theta=theta, layers=layers, seq_lens=(tokens,),
                        k_bits=3, v_bits=3, key_dtype=key_dtype, profile=profile, outlier_blocks=outliers,
                        elem_outlier_p=elem_p)
    return [
        w("panel_d128_g4_loguniform_bf16", 21, 128, 32, 8, 5e5, "loguniform", "bf16", 0, 0.01),
        w("panel_d128_g8_decay_jitter", 22, 128, 16, 2, 1e6, "decay_jitter"),
        w("panel_d128_g7_decay", 23, 128, 28, 4, 1e6, "decay"),
        w("panel_d64_g1_decay", 24, 64, 8, 8, 1e4, "decay"),
        w("panel_d256_g8_decay_jitter", 25, 256, 8, 1, 1e6, "decay_jitter"),
    ]


WORKLOADS = {w.name: w for w in (TINY, LLAMA8B_LAYER, QWEN3B_128K, QWEN3B_512K, QWEN7B_RAGGED)}


# ---------------------------------------------------------------- profiles

def sigma(wl: Workload, seq: int, layer: int, head: int) -> np.ndarray:
    """Per-block standard deviation sigma_j of the pre-RoPE keys of one KV head."""
    n = wl.n
    rng = _rng(wl, seq, layer, head, _STREAMS["profile"])
    j = np.arange(n, dtype=np.float64)
    if wl.profile == "decay":
        s = 0.05 ** (j / (n - 1))
    elif wl.profile == "decay_jitter":
        s = 0.05 ** (j / (n - 1)) * np.exp(rng.uniform(math.log(0.5), math.log(2.0), size=n))
    elif wl.profile == "loguniform":
        e = np.exp(rng.uniform(math.log(1e-3), math.log(1.0), size=n))
        s = np.sqrt(e / 2.0)
    else:
        raise ValueError(wl.profile)
    if wl.outlier_blocks:
        idx = rng.choice(n, size=wl.outlier_blocks, replace=False)
        s[idx] *= 8.0
    return s


def _coord_sigma(wl: Workload, s_block: np.ndarray) -> np.ndarray:
    return np.concatenate([s_block, s_block])          # half pairing: (j, j + d/2)


def _to_dtype(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 to the storage dtype, returned as fp32 holding the exact rounded values."""
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        u = x32.view(np.uint32).astype(np.uint64)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16       # nearest-even to bf16
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


def _rope_keys(x: np.ndarray, pos: np.ndarray, d: int, theta: float) -> np.ndarray:
    n = d // 2
    inv = np.power(float(theta), -2.0 * np.arange(n, dtype=np.float64) / d)
    ang = np.mod(pos.astype(np.float64)[:, None] * inv[None, :], 2.0 * math.pi)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :n], x[:, n:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


def keys(wl: Workload, seq: int, layer: int, head: int, t0: int, t1: int) -> np.ndarray:
    """Post-RoPE keys of tokens [t0, t1) of one KV head, fp32 array of dtype-exact values."""
    sb = _coord_sigma(wl, sigma(wl, seq, layer, head))
    out = np.empty((t1 - t0, wl.d), dtype=np.float32)
    for blk in range(t0 // GEN_BLOCK, -(-t1 // GEN_BLOCK)):
        b0 = blk * GEN_BLOCK
        rng = _rng(wl, seq, layer, head, _STREAMS["k"], blk)
        x = rng.standard_normal((GEN_BLOCK, wl.d)) * sb[None, :]
        if wl.elem_outlier_p > 0:
            orng = _rng(wl, seq, layer, head, _STREAMS["outl"], blk)
            hit = orng.random((GEN_BLOCK, wl.d)) < wl.elem_outlier_p
            x = np.where(hit, orng.standard_t(3.0, size=(GEN_BLOCK, wl.d)) * sb[None, :], x)
        lo, hi = max(t0, b0), min(t1, b0 + GEN_BLOCK)
        pos = np.arange(lo, hi)
        xr = _rope_keys(x[lo - b0:hi - b0], pos, wl.d, wl.theta)
        out[lo - t0:hi - t0] = _to_dtype(xr, wl.key_dtype)
    return out


def values(wl: Workload, seq: int, layer: int, head: int, t0: int, t1: int) -> np.ndarray:
    """Values of tokens [t0, t1) of one KV head, N(0, 1) rounded to the key dtype."""
    out = np.empty((t1 - t0, wl.d), dtype=np.float32)
    for blk in range(t0 // GEN_BLOCK, -(-t1 // GEN_BLOCK)):
        b0 = blk * GEN_BLOCK
        x = _rng(wl, seq, layer, head, _STREAMS["v"], blk).standard_normal((GEN_BLOCK, wl.d))
        lo, hi = max(t0, b0), min(t1, b0 + GEN_BLOCK)
        out[lo - t0:hi - t0] = _to_dtype(x[lo - b0:hi - b0], wl.key_dtype)
    return out


def queries(wl: Workload, seq: int, layer: int, step: int = 0) -> np.ndarray:
    """Pre-RoPE queries [h_q, d] (fp32); query head h follows KV head h // group's profile."""
    out = np.empty((wl.h_q, wl.d), dtype=np.float32)
    for h in range(wl.h_q):
        sb = _coord_sigma(wl, sigma(wl, seq, layer, h // wl.group))
        rng = _rng(wl, seq, layer, h, _STREAMS["q"], step)
        out[h] = (rng.standard_normal(wl.d) * sb).astype(np.float32)
    return out


def new_token(wl: Workload, seq: int, layer: int, head: int, step: int):
    """(key, value) of the token appended at decode step `step` (cache position len + step)."""
    t = wl.seq_lens[seq] + step
    return keys(wl, seq, layer, head, t, t + 1)[0], values(wl, seq, layer, head, t, t + 1)[0]


# ---------------------------------------------------------------- rotations

def haar(m: int, rng: np.random.Generator) -> np.ndarray:
    """Haar-distributed orthogonal m x m matrix (QR of a Gaussian matrix, signs fixed), fp64."""
    g = rng.standard_normal((m, m))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def rotation_bank(d: int, seed: int = 0) -> np.ndarray:
    """Concatenated fp32 matrices for m = 2, 4, ..., d (row-major), for the key width groups."""
    parts = []
    for m in range(2, d + 1, 2):
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(_STREAMS["rot"], m)))
        parts.append(haar(m, rng).astype(np.float32).reshape(-1))
    return np.concatenate(parts)


def rotation_v(d: int, seed: int = 0) -> np.ndarray:
    """fp32 d x d rotation for values."""
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(_STREAMS["rotv"], d)))
    return haar(d, rng).astype(np.float32)


# ---------------------------------------------------------------- bulk device generation

def keys_values_device(wl: Workload, seq: int, layer: int, head: int, t_len: int, device, seed: int = 0):
    """Bulk (keys, values) [t_len, d] generated on a torch device for throughput runs.

    Same recipe as ``keys``/``values`` (per-block sigma, RoPE at positions 0..t_len-1,
    N(0, 1) values) drawn with torch's generator, so the bytes differ from the numpy
    streams; used where only the shape and distribution matter.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(hash((wl.wid, seed, seq, layer, head)) & 0x7FFFFFFF)
    sb = torch.tensor(_coord_sigma(wl, sigma(wl, seq, layer, head)), dtype=torch.float64, device=device)
    x = torch.randn((t_len, wl.d), generator=g, device=device, dtype=torch.float64) * sb
    n = wl.n
    inv = torch.pow(torch.tensor(float(wl.theta), dtype=torch.float64, device=device),
                    -2.0 * torch.arange(n, dtype=torch.float64, device=device) / wl.d)
    pos = torch.arange(t_len, dtype=torch.float64, device=device)
    ang = torch.remainder(pos[:, None] * inv[None, :], 2.0 * math.pi)
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[:, :n], x[:, n:]
    k = torch.cat([a * c - b * s, a * s + b * c], dim=1)
    v = torch.randn((t_len, wl.d), generator=g, device=device, dtype=torch.float64)
    dt = torch.float32 if wl.key_dtype == "f32" else torch.bfloat16
    return k.to(dt), v.to(dt)


# ---------------------------------------------------------------- structured rotations

GIVENS_HEADER = 128      # header entries: one per even size m = 2 .. 256


def givens_layer_count(m: int) -> int:
    """Layers drawn for size m: 2 ceil(log2 m) - 1 (odd, so that a size-2 rotation is not a
    signed permutation: 1 for m = 2, 13 for m = 128)."""
    return 2 * max(1, (m - 1).bit_length()) - 1


def givens_bank(d: int, seed: int = 0) -> np.ndarray:
    """Random Givens-layer rotations for every even size m = 2 .. d, packed as uint32 [N, 4].

    Size m gets givens_layer_count(m) layers; a layer is a uniformly random perfect matching of
    the m coordinates (a random permutation read in pairs) and one angle per pair, uniform over
    pi/4 + k pi/2 (k = 0..3: an equal split of the pair's mass with a random sign pattern, which
    spreads sparse vectors as evenly as possible per layer), stored as fp32 cos and sin.  Layout: GIVENS_HEADER header rows, row m/2 - 1 =
    (first record row of size m, layer count, 0, 0) (zeros for sizes above d); then the
    records (a | b << 16, bits of cos, bits of sin, 0), size by size, layer by layer."""
    header = np.zeros((GIVENS_HEADER, 4), dtype=np.uint32)
    recs = []
    row = GIVENS_HEADER
    for m in range(2, d + 1, 2):
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(_STREAMS["givens"], m)))
        n_layers = givens_layer_count(m)
        header[m // 2 - 1] = (row, n_layers, 0, 0)
        for _ in range(n_layers):
            perm = rng.permutation(m)
            theta = math.pi / 4 + (math.pi / 2) * rng.integers(0, 4, size=m // 2)
            r = np.zeros((m // 2, 4), dtype=np.uint32)
            r[:, 0] = perm[0::2].astype(np.uint32) | (perm[1::2].astype(np.uint32) << 16)
            r[:, 1] = np.cos(theta).astype(np.float32).view(np.uint32)
            r[:, 2] = np.sin(theta).astype(np.float32).view(np.uint32)
            recs.append(r)
            row += m // 2
    return np.concatenate([header] + recs)

