"""GPU parity of the fp16 recent-key window (through the C ABI).

A cache with a window keeps the fp16 keys of each sequence's newest `window` tokens and
decode attention uses them in place of their quantized reconstruction.  Checked here:

* the window's contents, bit for bit, after prefills and appends of one and of several
  tokens (both append kernels), including appends longer than the window;
* decode logits and outputs against the oracle (2e-3 normwise per sequence and head), with
  windows shorter than, equal to and longer than the sequence, a window boundary inside a
  tile, the largest window, an empty sequence, bf16 inputs and interleaved pairing;
* the decode step with a window equals the append followed by the decode, bit for bit;
* the 128K-token layer with a 1024-token window at full size.
"""

import numpy as np
import pytest
import torch

from decode_attention_rope_amd import bgtq, synth
from oracle import allocate, energy, layout, quantize
from oracle import window as owin
from _ref import TOL, rel_err

pytestmark = pytest.mark.gpu


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _t(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(dtype)


_ROT = {}


def _rot(d):
    if d not in _ROT:
        bank, rv = synth.rotation_bank(d, seed=7), synth.rotation_v(d, seed=7)
        _ROT[d] = (bank, rv, bgtq.make_quantizer(_t(bank), _t(rv), d))
    return _ROT[d]


def _build(wl, pre, appends, w, kdt, pairing, cap=None):
    """Prefill pre[s] tokens of every sequence, then append `appends` (token counts) to every
    sequence with a non-empty prefill.  Returns the cache and the tokens' keys and values."""
    dev = _cuda()
    bank, rv, qz = _rot(wl.d)
    tdt = torch.bfloat16 if kdt == "bf16" else torch.float32
    total = [p + (sum(appends) if p else 0) for p in pre]
    cap = cap or -(-max(max(total), 1) // 64) * 64
    cache = bgtq.PackedCache(len(pre), wl.h_kv, wl.d, wl.budget, wl.v_bits, cap, pairing=pairing, device=dev,
                             window=w)
    kv = []
    for s, t_len in enumerate(total):
        k = np.stack([synth.keys(wl, s, 0, h, 0, t_len) for h in range(wl.h_kv)])
        v = np.stack([synth.values(wl, s, 0, h, 0, t_len) for h in range(wl.h_kv)])
        kv.append((torch.from_numpy(k).to(tdt).float().numpy(), torch.from_numpy(v).to(tdt).float().numpy()))
        if pre[s]:
            bgtq.bgtq_prefill(qz, cache, _t(k[:, :pre[s]], tdt), _t(v[:, :pre[s]], tdt), s)
    start = list(pre)
    for n in appends:
        for s in range(len(pre)):
            if pre[s]:
                k, v = kv[s]
                bgtq.bgtq_quantize_append(qz, cache, _t(k[:, start[s]:start[s] + n], tdt)[None],
                                          _t(v[:, start[s]:start[s] + n], tdt)[None], seq_begin=s)
                start[s] += n
    torch.cuda.synchronize()
    assert cache.lengths.tolist() == total and int(cache.status[0]) == 0
    return cache, kv, total


def _check_ring(cache, kv, total, w):
    ring = cache.k_window.cpu().numpy()
    for s, t_len in enumerate(total):
        k, _ = kv[s]
        lo, hi = owin.window_range(t_len, w)
        for t in range(lo, hi):
            want = np.clip(k[:, t], -65504, 65504).astype(np.float16).view(np.int16)
            np.testing.assert_array_equal(ring[s, :, t % w], want, err_msg=f"seq {s} token {t}")


def _check_decode(cache, kv, total, pre, wl, w, qdt, pairing):
    bank, rv, qz = _rot(wl.d)
    tq = torch.bfloat16 if qdt == "bf16" else torch.float32
    q = torch.from_numpy(np.stack([synth.queries(wl, s, 0) for s in range(len(total))])).to(tq).float().numpy()
    out, logits = bgtq.bgtq_decode_attention(qz, cache, _t(q, tq), wl.theta, logits=True)
    torch.cuda.synchronize()
    out, logits = out.cpu().numpy(), logits.cpu().numpy()
    g, worst = wl.group, 0.0
    for s, t_len in enumerate(total):
        if t_len == 0:
            assert not out[s].any()
            continue
        k, v = kv[s]
        for h in range(wl.h_kv):
            lay = layout.build(allocate.greedy(energy.block_energy(k[h, :pre[s]], pairing), wl.budget), pairing)
            kh = quantize.dequantize_keys(*quantize.quantize_keys(k[h], lay, bank), lay, bank)
            vh = quantize.dequantize_values(*quantize.quantize_values(v[h], rv, wl.v_bits), rv, wl.v_bits)
            o_ref, l_ref = owin.decode_head_group(q[s, h * g:(h + 1) * g], t_len - 1, wl.theta, kh, k[h], vh, w,
                                                  pairing=pairing)
            e_log = rel_err(logits[s, h * g:(h + 1) * g, :t_len], l_ref)
            e_out = rel_err(out[s, h * g:(h + 1) * g], o_ref)
            assert np.all(e_log <= TOL), f"seq {s} head {h}: logit error {e_log}"
            assert np.all(e_out <= TOL), f"seq {s} head {h}: output error {e_out}"
            worst = max(worst, float(e_log.max()), float(e_out.max()))
    _say(f"  worst rel err {worst:.2e}")


@pytest.mark.parametrize("d,h_q,h_kv,pre,appends,w,kdt,qdt,pairing", [
    (128, 16, 2, [300, 130, 1, 0], [1, 1, 5, 1], 64, "f32", "f32", 0),     # boundary inside a tile
    (64, 4, 4, [255, 64], [1], 100, "bf16", "bf16", 1),
    (256, 4, 1, [70], [3], 300, "f32", "f32", 0),                           # window longer than the sequence
    (128, 8, 1, [1000], [200], 1, "f32", "f32", 0),                         # one-token window, long append
    (128, 16, 2, [5000, 4096], [1], 4096, "bf16", "f32", 0),                # the largest window
])
def test_window_contents_and_decode(d, h_q, h_kv, pre, appends, w, kdt, qdt, pairing):
    _cuda()
    _say(f"window d={d} {h_q}/{h_kv} pre={pre} appends={appends} w={w} {kdt}/{qdt} pairing={pairing}")
    wl = synth.Workload("window", 95, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=tuple(pre), k_bits=3,
                        v_bits=2, key_dtype=kdt, profile="decay_jitter", outlier_blocks=2)
    cache, kv, total = _build(wl, pre, appends, w, kdt, pairing)
    _check_ring(cache, kv, total, w)
    _check_decode(cache, kv, total, pre, wl, w, qdt, pairing)


@pytest.mark.parametrize("d,h_q,h_kv,pre,w,kdt", [
    (128, 16, 2, [200, 63], 64, "f32"),
    (64, 8, 2, [129], 1000, "bf16"),
])
def test_decode_step_with_window_equals_append_then_decode(d, h_q, h_kv, pre, w, kdt):
    dev = _cuda()
    _say(f"window step d={d} {h_q}/{h_kv} pre={pre} w={w} {kdt}")
    steps = 3
    wl = synth.Workload("window_step", 96, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1,
                        seq_lens=tuple(p + steps for p in pre), k_bits=3, v_bits=3, key_dtype=kdt, profile="decay",
                        outlier_blocks=2)
    _, _, qz = _rot(d)
    tdt = torch.bfloat16 if kdt == "bf16" else torch.float32
    cap = -(-(max(pre) + steps) // 64) * 64
    caches = []
    kv = [(np.stack([synth.keys(wl, s, 0, h, 0, pre[s] + steps) for h in range(h_kv)]),
           np.stack([synth.values(wl, s, 0, h, 0, pre[s] + steps) for h in range(h_kv)])) for s in range(len(pre))]
    for _ in range(2):
        c = bgtq.PackedCache(len(pre), h_kv, d, wl.budget, wl.v_bits, cap, device=dev, window=w)
        for s, p in enumerate(pre):
            bgtq.bgtq_prefill(qz, c, _t(kv[s][0][:, :p], tdt), _t(kv[s][1][:, :p], tdt), s)
        caches.append(c)
    a, b = caches
    ws = [torch.zeros(bgtq.decode_workspace_bytes(len(pre), h_q, h_kv, d, cap), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    gen = torch.Generator().manual_seed(9)
    for step in range(steps):
        kn = torch.stack([_t(kv[s][0][:, pre[s] + step:pre[s] + step + 1], tdt) for s in range(len(pre))])
        vn = torch.stack([_t(kv[s][1][:, pre[s] + step:pre[s] + step + 1], tdt) for s in range(len(pre))])
        q = torch.randn((len(pre), h_q, d), generator=gen).to(dev)
        bgtq.bgtq_quantize_append(qz, a, kn.contiguous(), vn.contiguous())
        out_a, lg_a = bgtq.bgtq_decode_attention(qz, a, q, 1e6, logits=True, workspace=ws[0])
        out_b, lg_b = bgtq.bgtq_decode_step(qz, b, q, kn.contiguous(), vn.contiguous(), 1e6, logits=True,
                                            workspace=ws[1])
        torch.cuda.synchronize()
        assert a.lengths.tolist() == b.lengths.tolist()
        assert torch.equal(out_a, out_b), f"step {step}: outputs differ"
        torch.testing.assert_close(lg_a, lg_b, rtol=0, atol=0, equal_nan=True)
        assert torch.equal(a.k_window, b.k_window), f"step {step}: window differs"


def test_window_needs_the_matrix_core_decode():
    dev = _cuda()
    _, _, qz = _rot(128)
    cache = bgtq.PackedCache(1, 1, 128, 192, 3, 64, device=dev, window=16)
    with pytest.raises(bgtq.BgtqError) as e:
        bgtq.bgtq_decode_attention(qz, cache, torch.zeros((1, 16, 128), device=dev), 1e6)
    assert e.value.status == bgtq.ERR_UNSUPPORTED


def test_window_qwen3b_layer_128k_full_size():
    """The 128K-token layer (16 query / 2 KV heads, K3V3) with a 1024-token window: prefill
    131072 tokens, one decode step, every head against the oracle."""
    dev = _cuda()
    _say("window qwen3b 128K full size, w = 1024")
    wl, w = synth.QWEN3B_128K, 1024
    bank, rv, qz = _rot(128)
    t_len = wl.seq_lens[0] + 1
    cap = -(-t_len // 64) * 64
    cache = bgtq.PackedCache(1, wl.h_kv, wl.d, wl.budget, wl.v_bits, cap, device=dev, window=w)
    k = np.stack([synth.keys(wl, 0, 0, h, 0, t_len) for h in range(wl.h_kv)])
    v = np.stack([synth.values(wl, 0, 0, h, 0, t_len) for h in range(wl.h_kv)])
    bgtq.bgtq_prefill(qz, cache, _t(k[:, :-1]), _t(v[:, :-1]), 0)
    q = synth.queries(wl, 0, 0)
    out, logits = bgtq.bgtq_decode_step(qz, cache, _t(q[None]), _t(k[None, :, -1:]), _t(v[None, :, -1:]), wl.theta,
                                        logits=True)
    torch.cuda.synchronize()
    assert int(cache.lengths[0]) == t_len
    _check_ring(cache, [(k, v)], [t_len], w)
    out, logits = out.cpu().numpy()[0], logits.cpu().numpy()[0]
    g = wl.group
    for h in range(wl.h_kv):
        lay = layout.build(allocate.greedy(energy.block_energy(k[h, :-1]), wl.budget))
        kh = quantize.dequantize_keys(*quantize.quantize_keys(k[h], lay, bank), lay, bank)
        vh = quantize.dequantize_values(*quantize.quantize_values(v[h], rv, wl.v_bits), rv, wl.v_bits)
        o_ref, l_ref = owin.decode_head_group(q[h * g:(h + 1) * g], t_len - 1, wl.theta, kh, k[h], vh, w)
        e_log = rel_err(logits[h * g:(h + 1) * g, :t_len], l_ref)
        e_out = rel_err(out[h * g:(h + 1) * g], o_ref)
        _say(f"  kv head {h}: logit err {e_log.max():.2e}, output err {e_out.max():.2e}")
        assert np.all(e_log <= TOL) and np.all(e_out <= TOL)
