"""bgtq_prefill against the three calls it stands for (GPU).

The one-call prefill (energy partials, then the energies' final sums and the allocation in
one kernel, then the quantize-and-append) must equal bgtq_block_energy + bgtq_allocate_bits
+ bgtq_quantize_append bit for bit: energies, widths, layouts, every cache array, lengths
and the recent-key window.  Those three calls are checked against the oracle by
test_gpu_parity.py; the prefill path itself is what bgtq_prefill (and so every other
parity test) uses.
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


@pytest.mark.parametrize("d,k_bits,v_bits,t_len,kdt,pairing,rotation,window,b_min,b_max,seq", [
    (128, 3, 3, 1000, "f32", 0, "dense", 0, 0, 8, 0),
    (128, 2, 2, 257, "bf16", 1, "dense", 64, 1, 4, 1),
    (64, 3, 1, 3000, "f32", 0, "givens", 0, 0, 8, 2),
    (256, 3, 2, 129, "f32", 0, "givens", 100, 0, 8, 0),
    (128, 0, 3, 40, "f32", 0, "dense", 0, 0, 8, 1),
    (128, 3, 3, 70000, "f32", 0, "dense", 0, 0, 8, 0),
])
def test_prefill_equals_the_three_calls(d, k_bits, v_bits, t_len, kdt, pairing, rotation, window, b_min, b_max, seq):
    dev = _cuda()
    _say(f"prefill d={d} K{k_bits}V{v_bits} T={t_len} {kdt} pairing={pairing} {rotation} window={window} "
         f"b=[{b_min},{b_max}] seq={seq}")
    wl = synth.Workload("prefill", 100, d=d, h_q=4, h_kv=2, theta=1e4, layers=1, seq_lens=(t_len,), k_bits=k_bits,
                        v_bits=v_bits, key_dtype=kdt, profile="decay_jitter", outlier_blocks=2)
    tdt = torch.bfloat16 if kdt == "bf16" else torch.float32
    if rotation == "givens":
        qz = bgtq.make_quantizer(None, None, d, givens=_t(synth.givens_bank(d, seed=2).view(np.int32), torch.int32))
    else:
        qz = bgtq.make_quantizer(_t(synth.rotation_bank(d, seed=2)), _t(synth.rotation_v(d, seed=2)), d)
    k = _t(np.stack([synth.keys(wl, 0, 0, h, 0, t_len) for h in range(2)]), tdt)
    v = _t(np.stack([synth.values(wl, 0, 0, h, 0, t_len) for h in range(2)]), tdt)
    cap = -(-t_len // 64) * 64 + 64
    batch = max(seq + 1, 2)
    a = bgtq.PackedCache(batch, 2, d, wl.budget, v_bits, cap, pairing=pairing, device=dev, window=window)
    b = bgtq.PackedCache(batch, 2, d, wl.budget, v_bits, cap, pairing=pairing, device=dev, window=window)
    # the three calls
    e_a = bgtq.bgtq_block_energy(k, pairing)
    bgtq.bgtq_allocate_bits(e_a, wl.budget, b_min, b_max, pairing, widths_out=a.widths[seq], layouts_out=a.layouts[seq])
    bgtq.bgtq_quantize_append(qz, a, k.unsqueeze(0), v.unsqueeze(0), seq_begin=seq)
    # the one call
    e_b = torch.empty((2, d // 2), dtype=torch.float64, device=dev)
    bgtq.bgtq_prefill(qz, b, k, v, seq, b_min, b_max, energy_out=e_b)
    torch.cuda.synchronize()
    assert torch.equal(e_a, e_b)
    for name in ("widths", "layouts", "k_codes", "k_norms", "v_codes", "v_norms", "lengths", "status"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    if window:
        assert torch.equal(a.k_window, b.k_window)
    assert b.lengths.tolist() == [t_len if s == seq else 0 for s in range(batch)]
