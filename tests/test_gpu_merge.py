"""The decode merge's output contract (GPU).

The merge runs two workgroups per query head, and each adds its half of the result into `out`,
which the split pass clears first. So the output must not depend on what `out` held before
the call. Repeated calls must agree bit for bit: each element is the sum of exactly two terms,
which is the same in either order. Accuracy against the oracle is covered by
test_gpu_parity.py and test_gpu_givens.py; this file checks only these two properties.
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


def _t(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(dtype)


@pytest.mark.parametrize("rotation,d,h_q,h_kv,t_lens", [
    ("dense", 128, 16, 2, [3000, 70]),     # many splits per head; a short second sequence
    ("givens", 128, 16, 2, [3000, 70]),
    ("dense", 64, 8, 2, [1]),              # one token: a single split
    ("givens", 256, 4, 1, [700]),
])
def test_merge_output_ignores_prior_contents_and_repeats(rotation, d, h_q, h_kv, t_lens):
    dev = _cuda()
    print(f"merge contract {rotation} d={d} {h_q}/{h_kv} lens={t_lens}", flush=True)
    wl = synth.Workload("merge", 97, d=d, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay", outlier_blocks=2)
    if rotation == "dense":
        qz = bgtq.make_quantizer(_t(synth.rotation_bank(d, seed=7)), _t(synth.rotation_v(d, seed=7)), d)
    else:
        rec = synth.givens_bank(d, seed=7)
        qz = bgtq.make_quantizer(None, None, d, givens=torch.from_numpy(rec.view(np.int32)).to(dev))
    cap = -(-max(t_lens) // 64) * 64
    cache = bgtq.PackedCache(len(t_lens), h_kv, d, wl.budget, wl.v_bits, cap, device=dev)
    for s, n in enumerate(t_lens):
        k = np.stack([synth.keys(wl, s, 0, h, 0, n) for h in range(h_kv)])
        v = np.stack([synth.values(wl, s, 0, h, 0, n) for h in range(h_kv)])
        bgtq.bgtq_prefill(qz, cache, _t(k), _t(v), s)
    q = torch.randn((len(t_lens), h_q, d), generator=torch.Generator().manual_seed(5)).to(dev)
    ws = torch.zeros(bgtq.decode_workspace_bytes(len(t_lens), h_q, h_kv, d, cap), dtype=torch.uint8, device=dev)

    ref = torch.zeros((len(t_lens), h_q, d), dtype=torch.float32, device=dev)
    bgtq.bgtq_decode_attention(qz, cache, q, wl.theta, out=ref, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all() and ref.abs().max() > 0

    for fill in (float("nan"), 1e30, -3.0):
        out = torch.full_like(ref, fill)
        bgtq.bgtq_decode_attention(qz, cache, q, wl.theta, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"output depends on the prior contents of out (fill {fill})"
    assert int(cache.status.max()) == 0
