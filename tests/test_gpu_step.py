"""bgtq_decode_step against the two calls it stands for (GPU).

One decode step appends one key/value token to every sequence and attends with the query at
that token's position.  The fused call runs the append as one workgroup of the attention pass
(the split that reads the new token's tile waits for it) and advances the lengths in its merge
kernel; its results must equal, bit for bit,
bgtq_quantize_append(n_new = 1) followed by bgtq_decode_attention(q_pos = None): outputs,
logits, every cache array, lengths and status.  The append-then-decode path itself is checked
against the oracle by test_gpu_parity.py.
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


def _say(msg):
    print(msg, flush=True)


def _t(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(dtype)


def _cache(wl, prefill, cap, qz, kv, tdt, dev):
    cache = bgtq.PackedCache(len(prefill), wl.h_kv, wl.d, wl.budget, wl.v_bits, cap, device=dev)
    for s, n in enumerate(prefill):
        k, v = kv[s]
        bgtq.bgtq_prefill(qz, cache, _t(k[:, :max(n, 1)], tdt), _t(v[:, :max(n, 1)], tdt), s)
        if n == 0:     # allocation from one token, then an empty sequence
            cache.lengths[s] = 0
    return cache


@pytest.mark.parametrize("d,k_bits,v_bits,h_q,h_kv,prefill,steps,kv_dtype,q_dtype,extra_cap", [
    (128, 3, 3, 16, 2, [300, 0, 130], 3, "f32", "f32", 64),     # the model shape, an empty sequence
    (64, 2, 2, 8, 2, [63, 64], 3, "bf16", "bf16", 64),          # tile boundaries, bf16 inputs
    (256, 3, 4, 4, 1, [70], 2, "f32", "f32", 64),
    (128, 3, 3, 32, 2, [40], 2, "f32", "f32", 64),              # group of 16: vector-ALU path
    (128, 3, 3, 8, 1, [127], 3, "f32", "f32", 0),               # the second step fills, the third overflows
])
def test_decode_step_equals_append_then_decode(d, k_bits, v_bits, h_q, h_kv, prefill, steps, kv_dtype, q_dtype,
                                               extra_cap):
    dev = _cuda()
    _say(f"decode step d={d} K{k_bits}V{v_bits} {h_q}/{h_kv} prefill={prefill} steps={steps} {kv_dtype}/{q_dtype}")
    t_lens = [max(p, 1) + steps for p in prefill]
    cap = -(-(max(prefill) + 1) // 64) * 64 + extra_cap
    wl = synth.Workload("step", 91, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=k_bits, v_bits=v_bits, key_dtype=kv_dtype, profile="decay", outlier_blocks=2)
    bank, rv = synth.rotation_bank(d, seed=3), synth.rotation_v(d, seed=3)
    qz = bgtq.make_quantizer(_t(bank), _t(rv), d)
    kvt = torch.bfloat16 if kv_dtype == "bf16" else torch.float32
    qt = torch.bfloat16 if q_dtype == "bf16" else torch.float32
    kv = [(np.stack([synth.keys(wl, s, 0, h, 0, t_lens[s]) for h in range(h_kv)]),
           np.stack([synth.values(wl, s, 0, h, 0, t_lens[s]) for h in range(h_kv)])) for s in range(len(prefill))]
    a = _cache(wl, prefill, cap, qz, kv, kvt, dev)
    b = _cache(wl, prefill, cap, qz, kv, kvt, dev)
    ws_bytes = bgtq.decode_workspace_bytes(len(prefill), h_q, h_kv, d, cap)
    ws_a = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    ws_b = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    gen = torch.Generator().manual_seed(5)
    for step in range(steps):
        kn = torch.stack([_t(kv[s][0][:, prefill[s] + step:prefill[s] + step + 1], kvt) for s in range(len(prefill))])
        vn = torch.stack([_t(kv[s][1][:, prefill[s] + step:prefill[s] + step + 1], kvt) for s in range(len(prefill))])
        q = torch.randn((len(prefill), h_q, d), generator=gen).to(qt).to(dev)
        bgtq.bgtq_quantize_append(qz, a, kn.contiguous(), vn.contiguous())
        out_a, lg_a = bgtq.bgtq_decode_attention(qz, a, q, 1e6, logits=True, workspace=ws_a)
        out_b, lg_b = bgtq.bgtq_decode_step(qz, b, q, kn.contiguous(), vn.contiguous(), 1e6, logits=True,
                                            workspace=ws_b)
        torch.cuda.synchronize()
        assert a.lengths.tolist() == b.lengths.tolist(), f"step {step}"
        assert int(a.status[0]) == int(b.status[0]), f"step {step}"
        assert torch.equal(out_a, out_b), f"step {step}: outputs differ"
        torch.testing.assert_close(lg_a, lg_b, rtol=0, atol=0, equal_nan=True)
        for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
            assert torch.equal(getattr(a, name), getattr(b, name)), f"step {step}: {name}"
    if extra_cap == 0:
        assert int(b.status[0]) == 1 and b.lengths.tolist() == [cap]


def test_step_wait_that_gives_up_is_reported():
    """The attention pass waits for its own append with a bounded spin.  With the bound forced
    to zero from the host (the spin is skipped), the pass reports bit 1 in the cache's status;
    with the normal bound it does not.  No wait hangs either way."""
    dev = _cuda()
    d, h_q, h_kv, pre = 128, 16, 2, 130
    _say("decode step: bounded wait report")
    wl = synth.Workload("step_wait", 96, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=(pre + 2,),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay", outlier_blocks=2)
    bank, rv = synth.rotation_bank(d, seed=5), synth.rotation_v(d, seed=5)
    qz = bgtq.make_quantizer(_t(bank), _t(rv), d)
    k = np.stack([synth.keys(wl, 0, 0, h, 0, pre + 2) for h in range(h_kv)])
    v = np.stack([synth.values(wl, 0, 0, h, 0, pre + 2) for h in range(h_kv)])
    cache = bgtq.PackedCache(1, h_kv, d, wl.budget, wl.v_bits, 256, device=dev)
    bgtq.bgtq_prefill(qz, cache, _t(k[:, :pre]), _t(v[:, :pre]), 0)
    ws = torch.zeros(bgtq.decode_workspace_bytes(1, h_q, h_kv, d, 256), dtype=torch.uint8, device=dev)
    q = torch.randn((1, h_q, d), generator=torch.Generator().manual_seed(3)).to(dev)
    limit = bgtq.get_option(bgtq.OPT_STEP_WAIT_LIMIT)
    bgtq.set_option(bgtq.OPT_STEP_WAIT_LIMIT, 0)
    try:
        bgtq.bgtq_decode_step(qz, cache, q, _t(k[:, pre:pre + 1])[None].contiguous(),
                              _t(v[:, pre:pre + 1])[None].contiguous(), 1e6, workspace=ws)
        torch.cuda.synchronize()
    finally:
        bgtq.set_option(bgtq.OPT_STEP_WAIT_LIMIT, limit)
    assert int(cache.status[0]) & 2, "a wait that gave up was not reported"
    assert int(cache.lengths[0]) == pre + 1
    cache.status.zero_()
    bgtq.bgtq_decode_step(qz, cache, q, _t(k[:, pre + 1:pre + 2])[None].contiguous(),
                          _t(v[:, pre + 1:pre + 2])[None].contiguous(), 1e6, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.status[0]) == 0 and int(cache.lengths[0]) == pre + 2
