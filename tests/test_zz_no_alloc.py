"""bgtq_decode_step_noalloc against bgtq_decode_step (GPU).

The allocation-free step keeps its split partials and step flags in the library's per-GPU
scratch array instead of a caller workspace, and runs the same kernels.  Two calls in a row
(the second on a smaller cache, so its flags sit where the first call left partial results)
must each equal bgtq_decode_step bit for bit: outputs, logits, every cache array, lengths and
status.
"""

import numpy as np
import pytest
import torch

from decode_attention_rope_amd import bgtq, synth

pytestmark = pytest.mark.gpu


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _case(d, h_q, h_kv, prefill, k_bits, v_bits, seed):
    dev = _cuda()
    t_lens = [p + 1 for p in prefill]
    cap = -(-(max(prefill) + 1) // 64) * 64 + 64
    wl = synth.Workload("noalloc", seed, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=k_bits, v_bits=v_bits, key_dtype="f32", profile="decay", outlier_blocks=2)
    bank, rv = synth.rotation_bank(d, seed=seed), synth.rotation_v(d, seed=seed)
    qz = bgtq.make_quantizer(_t(bank), _t(rv), d)
    kv = [(np.stack([synth.keys(wl, s, 0, h, 0, t_lens[s]) for h in range(h_kv)]),
           np.stack([synth.values(wl, s, 0, h, 0, t_lens[s]) for h in range(h_kv)])) for s in range(len(prefill))]
    caches = []
    for _ in range(2):
        c = bgtq.PackedCache(len(prefill), h_kv, d, wl.budget, v_bits, cap, device=dev)
        for s, n in enumerate(prefill):
            bgtq.bgtq_prefill(qz, c, _t(kv[s][0][:, :n]), _t(kv[s][1][:, :n]), s)
        caches.append(c)
    kn = torch.stack([_t(kv[s][0][:, prefill[s]:prefill[s] + 1]) for s in range(len(prefill))]).contiguous()
    vn = torch.stack([_t(kv[s][1][:, prefill[s]:prefill[s] + 1]) for s in range(len(prefill))]).contiguous()
    q = torch.randn((len(prefill), h_q, d), generator=torch.Generator().manual_seed(seed)).to(dev)
    return qz, caches, kn, vn, q, cap


@pytest.mark.parametrize("cases", [[
    (128, 16, 2, [5000, 1300], 3, 3, 71),      # the serving shape, two sequences
    (64, 4, 1, [300], 2, 2, 72),               # then a smaller cache: fewer splits, other flag offset
]])
def test_noalloc_step_equals_decode_step(cases):
    for d, h_q, h_kv, prefill, k_bits, v_bits, seed in cases:
        print(f"noalloc step d={d} {h_q}/{h_kv} prefill={prefill} K{k_bits}V{v_bits}", flush=True)
        qz, (a, b), kn, vn, q, cap = _case(d, h_q, h_kv, prefill, k_bits, v_bits, seed)
        out_a, lg_a = bgtq.bgtq_decode_step(qz, a, q, kn, vn, 1e6, logits=True)
        lg_b = torch.full_like(lg_a, float("nan"))
        out_b = torch.empty_like(out_a)
        bgtq.bgtq_decode_step_noalloc(qz, b, q, kn, vn, 1e6, out=out_b, logits=lg_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b)
        for s, p in enumerate(prefill):
            assert torch.equal(lg_a[s, :, :p + 1], lg_b[s, :, :p + 1])
        assert torch.equal(a.lengths, b.lengths) and torch.equal(a.status, b.status)
        assert int(a.status[0]) == 0
        for name in ("k_codes", "k_norms", "v_codes", "v_norms", "widths", "layouts"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
