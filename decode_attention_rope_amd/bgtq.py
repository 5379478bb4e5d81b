"""Python binding of libbgtq.so (C ABI in include/bgtq.h).

Argument marshalling only: tensors are passed as device pointers, the stream is
torch's current HIP stream, and every step of the path runs in the library's
kernels.  torch is used for device memory and streams.  If the library is not
built the first call raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from dataclasses import dataclass

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbgtq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "bgtq.h")

OK, ERR_INVALID_ARG, ERR_BUDGET, ERR_CAPACITY, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP = range(7)
F32, BF16 = 0, 1
PAIR_HALF, PAIR_INTERLEAVED = 0, 1
ROT_DENSE, ROT_GIVENS = 0, 1
OPT_DECODE_KERNEL, OPT_STEP_WAIT_LIMIT = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20
TILE = 64
MAX_GROUPS = 8
LAYOUT_BYTES = 4096
MAX_WINDOW = 4096

_c = ctypes
_vp, _i32, _i64, _sz, _f32, _f64 = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_size_t, _c.c_float, _c.c_double


class BgtqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"bgtq status {status}: {message}")
        self.status = status


class Quantizer(_c.Structure):
    _fields_ = [("rot_bank", _vp), ("rot_v", _vp), ("rot_bank_t", _vp), ("rot_v_t", _vp), ("head_dim", _i32),
                ("rotation", _i32), ("givens", _vp)]


class CacheDesc(_c.Structure):
    _fields_ = [("batch", _i32), ("n_kv_heads", _i32), ("head_dim", _i32), ("k_width_sum", _i32),
                ("v_bits", _i32), ("capacity", _i64), ("pairing", _i32),
                ("k_codes", _vp), ("k_norms", _vp), ("v_codes", _vp), ("v_norms", _vp),
                ("lengths", _vp), ("widths", _vp), ("layouts", _vp), ("status", _vp),
                ("window", _i32), ("k_window", _vp)]


_SIGNATURES = {
    "bgtq_block_energy": (_i32, [_vp, _i32, _i32, _i64, _i32, _i64, _i64, _i32, _vp, _vp, _sz, _vp]),
    "bgtq_energy_workspace_bytes": (_sz, [_i32, _i64, _i32]),
    "bgtq_rotation_bank_floats": (_sz, [_i32]),
    "bgtq_transpose_rotations": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp]),
    "bgtq_allocate_bits": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "bgtq_quantize_append": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _vp]),
    "bgtq_decode_attention": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp, _f64, _f32, _vp, _vp, _vp, _sz, _vp]),
    "bgtq_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i64]),
    "bgtq_decode_step": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _f64, _f32, _vp, _vp, _vp,
                                _sz, _vp]),
    "bgtq_prefill": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _sz, _vp]),
    "bgtq_prefill_workspace_bytes": (_sz, [_i32, _i64, _i32]),
    "bgtq_logit_error": (_i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64,
                                _i32, _f64, _f32, _vp, _vp, _vp, _sz, _vp]),
    "bgtq_logit_error_workspace_bytes": (_sz, [_i32, _i32, _i64]),
    "bgtq_cache_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i64, _vp]),
    "bgtq_codebook": (_i32, [_i32, _vp, _vp, _vp]),
    "bgtq_init": (_i32, []),
    "bgtq_set_option": (_i32, [_i32, _i64]),
    "bgtq_get_option": (_i64, [_i32]),
    "bgtq_decode_step_noalloc": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _f64, _f32, _vp,
                                        _vp, _vp]),
    "bgtq_status_string": (_c.c_char_p, [_i32]),
    "bgtq_last_error": (_c.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_attention_rope_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def header_functions() -> list:
    """Names of the functions include/bgtq.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(bgtq_[a-z_0-9]+)\s*\(", text, re.M)))


def _check(status: int) -> None:
    if status != OK:
        raise BgtqError(status, lib().bgtq_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ host-only helpers

def codebook(bits: int):
    """(thresholds fp32, centroids fp32, fl32(D(bits)) as fp64) of the library's frozen tables."""
    n = 1 << bits
    thr = np.zeros(max(n - 1, 1), dtype=np.float32)
    cen = np.zeros(n, dtype=np.float32)
    dist = _c.c_double()
    _check(lib().bgtq_codebook(bits, thr.ctypes.data, cen.ctypes.data, _c.addressof(dist)))
    return (thr[:n - 1], cen, dist.value) if bits else (thr[:0], cen[:0], dist.value)


def cache_bytes(batch, n_kv_heads, head_dim, k_width_sum, v_bits, capacity):
    out4 = (_sz * 4)()
    total = lib().bgtq_cache_bytes(batch, n_kv_heads, head_dim, k_width_sum, v_bits, capacity, out4)
    if total == 0:
        raise BgtqError(ERR_INVALID_ARG, "invalid cache geometry")
    return total, tuple(out4)


def decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, capacity) -> int:
    return int(lib().bgtq_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, capacity))


def init() -> None:
    _check(lib().bgtq_init())


def set_option(option: int, value: int) -> None:
    """Process-wide test/diagnosis option (OPT_DECODE_KERNEL: 1 forces the vector-ALU decode,
    2 the tiled matrix-core pass; OPT_STEP_WAIT_LIMIT: bound of a decode step's wait for its
    append)."""
    _check(lib().bgtq_set_option(option, value))


def get_option(option: int) -> int:
    return int(lib().bgtq_get_option(option))


# ------------------------------------------------------------------ device objects

def make_quantizer(rot_bank: torch.Tensor | None, rot_v: torch.Tensor | None, head_dim: int,
                   givens: torch.Tensor | None = None):
    """C descriptor of the rotations (kept alive with it).  Dense: the Haar bank and the value
    rotation, whose transposed copies the library writes.  Structured: `givens`, the packed
    Givens-layer records (uint32 [rows, 4] bits in an int32 tensor)."""
    if givens is not None:
        if givens.dtype != torch.int32 or givens.dim() != 2 or givens.shape[1] != 4 or not givens.is_contiguous():
            raise ValueError("givens must be a contiguous int32 [rows, 4] tensor")
        q = Quantizer(None, None, None, None, head_dim, ROT_GIVENS, givens.data_ptr())
        q._keep = (givens,)
        return q
    n = int(lib().bgtq_rotation_bank_floats(head_dim))
    if n == 0 or rot_bank.numel() != n or rot_v.numel() != head_dim * head_dim:
        raise ValueError("rotation bank / value rotation do not match head_dim")
    if rot_bank.dtype != torch.float32 or rot_v.dtype != torch.float32:
        raise ValueError("rotations must be float32")
    rot_bank, rot_v = rot_bank.contiguous(), rot_v.contiguous()
    bank_t, rv_t = torch.empty_like(rot_bank), torch.empty_like(rot_v)
    _check(lib().bgtq_transpose_rotations(rot_bank.data_ptr(), rot_v.data_ptr(), head_dim, bank_t.data_ptr(),
                                          rv_t.data_ptr(), _stream()))
    q = Quantizer(rot_bank.data_ptr(), rot_v.data_ptr(), bank_t.data_ptr(), rv_t.data_ptr(), head_dim, ROT_DENSE,
                  None)
    q._keep = (rot_bank, rot_v, bank_t, rv_t)
    return q


@dataclass
class PackedCache:
    """Device memory of one layer's packed cache (allocated with torch, zero-filled)."""
    batch: int
    n_kv_heads: int
    head_dim: int
    k_width_sum: int
    v_bits: int
    capacity: int
    pairing: int = PAIR_HALF
    device: str = "cuda"
    window: int = 0           # fp16 recent-key window in tokens (0: none)

    def __post_init__(self):
        _, (kc, kn, vc, vn) = cache_bytes(self.batch, self.n_kv_heads, self.head_dim, self.k_width_sum,
                                          self.v_bits, self.capacity)
        dev = torch.device(self.device)
        self.k_codes = torch.zeros(max(kc, 16), dtype=torch.uint8, device=dev)
        self.k_norms = torch.zeros(kn // 2, dtype=torch.int16, device=dev)
        self.v_codes = torch.zeros(vc, dtype=torch.uint8, device=dev)
        self.v_norms = torch.zeros(vn // 2, dtype=torch.int16, device=dev)
        self.lengths = torch.zeros(self.batch, dtype=torch.int32, device=dev)
        self.widths = torch.zeros((self.batch, self.n_kv_heads, self.head_dim // 2), dtype=torch.uint8, device=dev)
        self.layouts = torch.zeros((self.batch, self.n_kv_heads, LAYOUT_BYTES), dtype=torch.uint8, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.k_chunks = -(-2 * self.k_width_sum // 128)
        # fp16 keys of the newest `window` tokens, token t at slot t % window (as uint16 bits)
        self.k_window = (torch.zeros((self.batch, self.n_kv_heads, self.window, self.head_dim), dtype=torch.int16,
                                     device=dev) if self.window > 0 else None)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.k_codes, self.k_norms, self.v_codes, self.v_norms))

    def desc(self) -> CacheDesc:
        return CacheDesc(self.batch, self.n_kv_heads, self.head_dim, self.k_width_sum, self.v_bits,
                         self.capacity, self.pairing, self.k_codes.data_ptr(), self.k_norms.data_ptr(),
                         self.v_codes.data_ptr(), self.v_norms.data_ptr(), self.lengths.data_ptr(),
                         self.widths.data_ptr(), self.layouts.data_ptr(), self.status.data_ptr(), self.window,
                         _ptr(self.k_window))

    def region(self, seq: int, head: int) -> dict:
        """Host copies of one (sequence, KV head) region, shaped like the oracle's pack_region."""
        h = seq * self.n_kv_heads + head
        tiles = self.capacity // TILE
        kcs = tiles * self.k_chunks * TILE * 16
        kns = tiles * MAX_GROUPS * TILE
        vcs = tiles * self.head_dim * 8 * self.v_bits
        vns = tiles * TILE
        return {
            "k_codes": self.k_codes[h * kcs:(h + 1) * kcs].cpu().numpy(),
            "k_norms": self.k_norms[h * kns:(h + 1) * kns].cpu().numpy().view(np.float16),
            "v_codes": self.v_codes[h * vcs:(h + 1) * vcs].cpu().numpy(),
            "v_norms": self.v_norms[h * vns:(h + 1) * vns].cpu().numpy().view(np.float16),
        }


# ------------------------------------------------------------------ the four calls

def bgtq_block_energy(keys: torch.Tensor, pairing: int = PAIR_HALF) -> torch.Tensor:
    """keys [n_heads, n_tokens, head_dim] (fp32/bf16, last dim contiguous) -> energy fp64 [n_heads, head_dim/2]."""
    if keys.dim() != 3 or keys.stride(2) != 1:
        raise ValueError("keys must be [n_heads, n_tokens, head_dim] with a contiguous last dimension")
    h, t, d = keys.shape
    out = torch.empty((h, d // 2), dtype=torch.float64, device=keys.device)
    ws_bytes = lib().bgtq_energy_workspace_bytes(h, t, d)
    ws = torch.empty(max(int(ws_bytes), 8), dtype=torch.uint8, device=keys.device)
    _check(lib().bgtq_block_energy(keys.data_ptr(), _dtype_code(keys), h, t, d, keys.stride(0), keys.stride(1),
                                   pairing, out.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return out


def bgtq_allocate_bits(energy: torch.Tensor, k_width_sum: int, b_min: int = 0, b_max: int = 8,
                       pairing: int = PAIR_HALF, widths_out=None, layouts_out=None):
    """energy fp64 [n_heads, n] -> (widths uint8 [n_heads, n], layouts uint8 [n_heads, 2048])."""
    if energy.dtype != torch.float64 or not energy.is_contiguous():
        raise ValueError("energy must be contiguous fp64")
    e2 = energy.reshape(-1, energy.shape[-1])
    h, n = e2.shape
    widths = widths_out if widths_out is not None else torch.empty((h, n), dtype=torch.uint8, device=energy.device)
    lay = layouts_out if layouts_out is not None else torch.empty((h, LAYOUT_BYTES), dtype=torch.uint8,
                                                                  device=energy.device)
    _check(lib().bgtq_allocate_bits(e2.data_ptr(), h, 2 * n, k_width_sum, b_min, b_max, pairing,
                                    widths.data_ptr(), lay.data_ptr(), _stream()))
    return widths, lay


def bgtq_quantize_append(quantizer: Quantizer, cache: PackedCache, keys: torch.Tensor, values: torch.Tensor,
                         seq_begin: int = 0) -> None:
    """keys, values [n_seqs, n_kv_heads, n_new, head_dim] (same strides) appended to sequences seq_begin.."""
    if keys.shape != values.shape or keys.stride() != values.stride() or keys.dtype != values.dtype:
        raise ValueError("keys and values must have the same shape, strides and dtype")
    if keys.dim() != 4 or keys.stride(3) != 1:
        raise ValueError("keys must be [n_seqs, n_kv_heads, n_new, head_dim] with a contiguous last dimension")
    n_seqs, hk, n_new, d = keys.shape
    if hk != cache.n_kv_heads or d != cache.head_dim:
        raise ValueError("keys do not match the cache geometry")
    desc = cache.desc()
    _check(lib().bgtq_quantize_append(_c.byref(quantizer), _c.byref(desc), seq_begin, n_seqs, keys.data_ptr(),
                                      values.data_ptr(), _dtype_code(keys), n_new, keys.stride(0), keys.stride(1),
                                      keys.stride(2), _stream()))


def bgtq_prefill(quantizer: Quantizer, cache: PackedCache, keys: torch.Tensor, values: torch.Tensor, seq: int,
                 b_min: int = 0, b_max: int = 8, energy_out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> None:
    """keys, values [n_kv_heads, T, head_dim] (same strides, last dim contiguous) of sequence `seq`:
    energies, widths and layouts, and the quantize-and-append of the T tokens, in one call."""
    if keys.shape != values.shape or keys.stride() != values.stride() or keys.dtype != values.dtype:
        raise ValueError("keys and values must have the same shape, strides and dtype")
    if keys.dim() != 3 or keys.stride(2) != 1:
        raise ValueError("keys must be [n_kv_heads, n_tokens, head_dim] with a contiguous last dimension")
    h, t, d = keys.shape
    if h != cache.n_kv_heads or d != cache.head_dim:
        raise ValueError("keys do not match the cache geometry")
    if energy_out is not None and (energy_out.dtype != torch.float64 or energy_out.numel() != h * (d // 2)):
        raise ValueError("energy_out must be fp64 [n_kv_heads, head_dim/2]")
    if workspace is None:
        workspace = torch.empty(max(int(lib().bgtq_prefill_workspace_bytes(h, t, d)), 8), dtype=torch.uint8,
                                device=keys.device)
    desc = cache.desc()
    _check(lib().bgtq_prefill(_c.byref(quantizer), _c.byref(desc), seq, keys.data_ptr(), values.data_ptr(),
                              _dtype_code(keys), t, keys.stride(0), keys.stride(1), b_min, b_max, _ptr(energy_out),
                              workspace.data_ptr(), workspace.numel(), _stream()))


def bgtq_decode_attention(quantizer: Quantizer, cache: PackedCache, q: torch.Tensor, rope_theta: float,
                          q_pos: torch.Tensor | None = None, softmax_scale: float | None = None,
                          out: torch.Tensor | None = None, logits: bool | torch.Tensor = False,
                          workspace: torch.Tensor | None = None):
    """q [batch, n_q_heads, head_dim] pre-RoPE -> out fp32 [batch, n_q_heads, head_dim] (and logits if asked)."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, n_q_heads, head_dim] tensor")
    b, hq, d = q.shape
    if b != cache.batch or d != cache.head_dim:
        raise ValueError("q does not match the cache geometry")
    if q_pos is not None and (q_pos.dtype != torch.int64 or q_pos.numel() != b):
        raise ValueError("q_pos must be int64 [batch]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
    lg = None
    if isinstance(logits, torch.Tensor):
        lg = logits
    elif logits:
        lg = torch.full((b, hq, cache.capacity), float("nan"), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.zeros(decode_workspace_bytes(b, hq, cache.n_kv_heads, d, cache.capacity),
                                dtype=torch.uint8, device=q.device)
    desc = cache.desc()
    _check(lib().bgtq_decode_attention(_c.byref(quantizer), _c.byref(desc), hq, q.data_ptr(), _dtype_code(q),
                                       _ptr(q_pos), float(rope_theta), float(scale), out.data_ptr(), _ptr(lg),
                                       workspace.data_ptr(), workspace.numel(), _stream()))
    return (out, lg) if logits is not False else out


def bgtq_decode_step(quantizer: Quantizer, cache: PackedCache, q: torch.Tensor, k_new: torch.Tensor,
                     v_new: torch.Tensor, rope_theta: float, softmax_scale: float | None = None,
                     out: torch.Tensor | None = None, logits: bool | torch.Tensor = False,
                     workspace: torch.Tensor | None = None):
    """Append one token per sequence (k_new, v_new [batch, n_kv_heads, 1, head_dim], same strides)
    and attend with q [batch, n_q_heads, head_dim] at its position, in one call."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, n_q_heads, head_dim] tensor")
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same shape, strides and dtype")
    b, hq, d = q.shape
    if k_new.dim() != 4 or k_new.shape[0] != b or k_new.shape[1] != cache.n_kv_heads or k_new.shape[2] != 1 \
            or k_new.shape[3] != d or k_new.stride(3) != 1:
        raise ValueError("k_new must be [batch, n_kv_heads, 1, head_dim] with a contiguous last dimension")
    if b != cache.batch or d != cache.head_dim:
        raise ValueError("q does not match the cache geometry")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
    lg = None
    if isinstance(logits, torch.Tensor):
        lg = logits
    elif logits:
        lg = torch.full((b, hq, cache.capacity), float("nan"), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.zeros(decode_workspace_bytes(b, hq, cache.n_kv_heads, d, cache.capacity),
                                dtype=torch.uint8, device=q.device)
    desc = cache.desc()
    _check(lib().bgtq_decode_step(_c.byref(quantizer), _c.byref(desc), hq, q.data_ptr(), _dtype_code(q),
                                  k_new.data_ptr(), v_new.data_ptr(), _dtype_code(k_new), k_new.stride(0),
                                  k_new.stride(1), float(rope_theta), float(scale), out.data_ptr(), _ptr(lg),
                                  workspace.data_ptr(), workspace.numel(), _stream()))
    return (out, lg) if logits is not False else out


def bgtq_decode_step_noalloc(quantizer: Quantizer, cache: PackedCache, q: torch.Tensor, k_new: torch.Tensor,
                             v_new: torch.Tensor, rope_theta: float, softmax_scale: float | None = None,
                             out: torch.Tensor | None = None, logits: torch.Tensor | None = None):
    """bgtq_decode_step without a workspace (the library's per-GPU scratch array holds it); `out`
    and `logits` (fp32 [batch, n_q_heads, capacity] or None) are caller-provided, so that a
    caller who must not allocate can pass buffers it already holds."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, n_q_heads, head_dim] tensor")
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same shape, strides and dtype")
    b, hq, d = q.shape
    if k_new.dim() != 4 or k_new.shape[0] != b or k_new.shape[1] != cache.n_kv_heads or k_new.shape[2] != 1 \
            or k_new.shape[3] != d or k_new.stride(3) != 1:
        raise ValueError("k_new must be [batch, n_kv_heads, 1, head_dim] with a contiguous last dimension")
    if b != cache.batch or d != cache.head_dim:
        raise ValueError("q does not match the cache geometry")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
    desc = cache.desc()
    _check(lib().bgtq_decode_step_noalloc(_c.byref(quantizer), _c.byref(desc), hq, q.data_ptr(), _dtype_code(q),
                                          k_new.data_ptr(), v_new.data_ptr(), _dtype_code(k_new), k_new.stride(0),
                                          k_new.stride(1), float(rope_theta), float(scale), out.data_ptr(),
                                          _ptr(logits), _stream()))
    return out


def logit_error_workspace_bytes(batch, n_q_heads, capacity) -> int:
    return int(lib().bgtq_logit_error_workspace_bytes(batch, n_q_heads, capacity))


def bgtq_logit_error(q: torch.Tensor, keys: torch.Tensor, lengths: torch.Tensor, logits: torch.Tensor,
                     rope_theta: float, softmax_scale: float | None = None, q_pos: torch.Tensor | None = None,
                     pairing: int = PAIR_HALF, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Mean |logits - exact logits| per (sequence, query head), fp64 [batch, n_q_heads].

    q [batch, n_q_heads, head_dim] pre-RoPE; keys [batch, n_kv_heads, tokens, head_dim] post-RoPE
    (last dimension contiguous); lengths int32 [batch]; logits fp32 [batch, n_q_heads, capacity]."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, n_q_heads, head_dim] tensor")
    b, hq, d = q.shape
    if keys.dim() != 4 or keys.shape[0] != b or keys.shape[3] != d or keys.stride(3) != 1:
        raise ValueError("keys must be [batch, n_kv_heads, tokens, head_dim] with a contiguous last dimension")
    if logits.dim() != 3 or logits.shape[:2] != (b, hq) or not logits.is_contiguous() \
            or logits.dtype != torch.float32:
        raise ValueError("logits must be contiguous fp32 [batch, n_q_heads, capacity]")
    if lengths.dtype != torch.int32 or lengths.numel() != b:
        raise ValueError("lengths must be int32 [batch]")
    if q_pos is not None and (q_pos.dtype != torch.int64 or q_pos.numel() != b):
        raise ValueError("q_pos must be int64 [batch]")
    cap = logits.shape[2]
    if keys.shape[2] < cap:
        raise ValueError("keys must hold capacity tokens (only those below lengths are read)")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    if out is None:
        out = torch.empty((b, hq), dtype=torch.float64, device=q.device)
    if workspace is None:
        workspace = torch.empty(logit_error_workspace_bytes(b, hq, cap), dtype=torch.uint8, device=q.device)
    _check(lib().bgtq_logit_error(q.data_ptr(), _dtype_code(q), _ptr(q_pos), keys.data_ptr(), _dtype_code(keys), b,
                                  hq, keys.shape[1], d, keys.stride(0), keys.stride(1), keys.stride(2),
                                  lengths.data_ptr(), cap, pairing, float(rope_theta), float(scale),
                                  logits.data_ptr(), out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                  _stream()))
    return out
