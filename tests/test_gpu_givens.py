"""GPU parity of the structured (Givens-layer) rotation kind, through the C ABI.

* Bit-exact against the oracle: every packed byte and norm after prefills and appends of
  one and of many tokens (the two append kernels), several head dims and budgets.
* Within 2e-3 normwise per (sequence, head): decode logits and outputs, on the matrix-core
  path, the vector-ALU path (groups of 16) and with a recent-key window.
* The decode step with structured rotations equals the append followed by the decode.
"""

import numpy as np
import pytest
import torch

from decode_attention_rope_amd import bgtq, synth
from oracle import quantize
from oracle import window as owin
from _ref import TOL, assert_region_equal, decode_reference, head_reference, rel_err

pytestmark = pytest.mark.gpu


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _t(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(dtype)


_Q = {}


def _quantizer(d):
    """(oracle rotations, library quantizer) for head dim d."""
    if d not in _Q:
        rec = synth.givens_bank(d, seed=11)
        dev_rec = torch.from_numpy(rec.view(np.int32)).to("cuda:0")
        _Q[d] = (quantize.Givens(rec), bgtq.make_quantizer(None, None, d, givens=dev_rec))
    return _Q[d]


@pytest.mark.parametrize("d,k_bits,v_bits,appends", [
    (128, 3, 3, [100, 1, 37, 64, 5]),
    (64, 3, 1, [1, 1, 70, 33]),
    (256, 3, 2, [129, 1]),
    (128, 8, 8, [65]),
    (128, 0, 3, [40, 1]),
    (128, 2, 2, [300]),
])
def test_quantize_append_bytes_bit_exact(d, k_bits, v_bits, appends):
    dev = _cuda()
    _say(f"givens append d={d} K{k_bits}V{v_bits} appends={appends}")
    giv, qz = _quantizer(d)
    t_len = sum(appends)
    cap = -(-t_len // 64) * 64 + 64
    wl = synth.Workload("givens_append", 97, d=d, h_q=4, h_kv=2, theta=1e4, layers=1, seq_lens=(t_len,),
                        k_bits=k_bits, v_bits=v_bits, key_dtype="f32", profile="decay_jitter", outlier_blocks=2)
    k = np.stack([synth.keys(wl, 0, 0, h, 0, t_len) for h in range(2)])
    v = np.stack([synth.values(wl, 0, 0, h, 0, t_len) for h in range(2)])
    cache = bgtq.PackedCache(1, 2, d, wl.budget, v_bits, cap, device=dev)
    e = bgtq.bgtq_block_energy(_t(k))
    bgtq.bgtq_allocate_bits(e, wl.budget, widths_out=cache.widths[0], layouts_out=cache.layouts[0])
    start = 0
    for n in appends:
        bgtq.bgtq_quantize_append(qz, cache, _t(k[:, start:start + n])[None], _t(v[:, start:start + n])[None])
        start += n
    torch.cuda.synchronize()
    assert int(cache.lengths[0]) == t_len and int(cache.status[0]) == 0
    for h in range(2):
        ref = head_reference(k[h], v[h], wl.budget, v_bits, giv, giv, cap)
        assert_region_equal(cache.region(0, h), ref["region"], t_len, ref["layout"], v_bits, d)


def _decode_case(wl, t_lens, kdt=torch.float32, window=0, valu=False):
    dev = _cuda()
    giv, qz = _quantizer(wl.d)
    d, h_kv, g = wl.d, wl.h_kv, wl.group
    cap = -(-max(t_lens) // 64) * 64
    cache = bgtq.PackedCache(len(t_lens), h_kv, d, wl.budget, wl.v_bits, cap, device=dev, window=window)
    kv = []
    for s, t_len in enumerate(t_lens):
        k = np.stack([synth.keys(wl, s, 0, h, 0, t_len) for h in range(h_kv)])
        v = np.stack([synth.values(wl, s, 0, h, 0, t_len) for h in range(h_kv)])
        kv.append((torch.from_numpy(k).to(kdt).float().numpy(), torch.from_numpy(v).to(kdt).float().numpy()))
        bgtq.bgtq_prefill(qz, cache, _t(k, kdt), _t(v, kdt), s)
    q = np.stack([synth.queries(wl, s, 0) for s in range(len(t_lens))])
    out, logits = bgtq.bgtq_decode_attention(qz, cache, _t(q), wl.theta, logits=True)
    torch.cuda.synchronize()
    out, logits = out.cpu().numpy(), logits.cpu().numpy()
    worst = 0.0
    for s, t_len in enumerate(t_lens):
        k, v = kv[s]
        for h in range(h_kv):
            ref = head_reference(k[h], v[h], wl.budget, wl.v_bits, giv, giv, cap)
            if window:
                o_ref, l_ref = owin.decode_head_group(q[s, h * g:(h + 1) * g], t_len - 1, wl.theta, ref["k_hat"], k[h],
                                                      ref["v_hat"], window)
            else:
                o_ref, l_ref = decode_reference(q[s, h * g:(h + 1) * g], t_len - 1, wl.theta, ref)
            e_log = rel_err(logits[s, h * g:(h + 1) * g, :t_len], l_ref)
            e_out = rel_err(out[s, h * g:(h + 1) * g], o_ref)
            assert np.all(e_log <= TOL), f"seq {s} head {h}: logit error {e_log}"
            assert np.all(e_out <= TOL), f"seq {s} head {h}: output error {e_out}"
            worst = max(worst, float(e_log.max()), float(e_out.max()))
    _say(f"  worst rel err {worst:.2e}")


@pytest.mark.parametrize("d,h_q,h_kv,t_lens,kdt,window", [
    (128, 14, 2, [1000, 3, 129], torch.float32, 0),       # group 7
    (128, 16, 2, [700], torch.bfloat16, 0),
    (64, 4, 1, [256, 65], torch.float32, 0),
    (256, 8, 2, [300], torch.float32, 0),
    (128, 32, 2, [500, 64], torch.float32, 0),             # group 16: the vector-ALU kernels
    (128, 16, 2, [900, 40], torch.float32, 128),           # with a recent-key window
])
def test_decode_parity(d, h_q, h_kv, t_lens, kdt, window):
    _say(f"givens decode d={d} {h_q}/{h_kv} lens={t_lens} {kdt} window={window}")
    wl = synth.Workload("givens_decode", 98, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay", outlier_blocks=2)
    _decode_case(wl, t_lens, kdt, window)


@pytest.mark.parametrize("d,h_q,pre", [(128, 16, [200, 63]), (256, 4, [70]),
                                       (128, 16, [131072])])   # full size: 127 split workgroups per KV head
def test_decode_step_equals_append_then_decode(d, h_q, pre):
    dev = _cuda()
    _say(f"givens step d={d} h_q={h_q} pre={pre}")
    giv, qz = _quantizer(d)
    h_kv, steps = 2 if h_q > 4 else 1, 3
    wl = synth.Workload("givens_step", 99, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1,
                        seq_lens=tuple(p + steps for p in pre), k_bits=3, v_bits=3, key_dtype="f32", profile="decay",
                        outlier_blocks=2)
    cap = -(-(max(pre) + steps) // 64) * 64
    kv = [(np.stack([synth.keys(wl, s, 0, h, 0, pre[s] + steps) for h in range(h_kv)]),
           np.stack([synth.values(wl, s, 0, h, 0, pre[s] + steps) for h in range(h_kv)])) for s in range(len(pre))]
    caches = []
    for _ in range(2):
        c = bgtq.PackedCache(len(pre), h_kv, d, wl.budget, wl.v_bits, cap, device=dev)
        for s, p in enumerate(pre):
            bgtq.bgtq_prefill(qz, c, _t(kv[s][0][:, :p]), _t(kv[s][1][:, :p]), s)
        caches.append(c)
    a, b = caches
    ws = [torch.zeros(bgtq.decode_workspace_bytes(len(pre), h_q, h_kv, d, cap), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    gen = torch.Generator().manual_seed(13)
    for step in range(steps):
        kn = torch.stack([_t(kv[s][0][:, pre[s] + step:pre[s] + step + 1]) for s in range(len(pre))])
        vn = torch.stack([_t(kv[s][1][:, pre[s] + step:pre[s] + step + 1]) for s in range(len(pre))])
        q = torch.randn((len(pre), h_q, d), generator=gen).to(dev)
        bgtq.bgtq_quantize_append(qz, a, kn.contiguous(), vn.contiguous())
        out_a, lg_a = bgtq.bgtq_decode_attention(qz, a, q, 1e6, logits=True, workspace=ws[0])
        out_b, lg_b = bgtq.bgtq_decode_step(qz, b, q, kn.contiguous(), vn.contiguous(), 1e6, logits=True,
                                            workspace=ws[1])
        torch.cuda.synchronize()
        assert a.lengths.tolist() == b.lengths.tolist()
        assert torch.equal(out_a, out_b), f"step {step}: outputs differ"
        torch.testing.assert_close(lg_a, lg_b, rtol=0, atol=0, equal_nan=True)
        for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
            assert torch.equal(getattr(a, name), getattr(b, name)), f"step {step}: {name}"
