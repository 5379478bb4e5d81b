"""Key-only RoPE logit-error diagnostic: Block-GTQ against uniform TQ-MSE at a matched budget.

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: with only the keys quantized,
at 2 and 3 bits per coordinate, Block-GTQ is reported to lower the per-layer mean absolute
error of the RoPE query-key logits against uniform TQ-MSE with the same budget, in every
layer compared.  This module runs that comparison on synthetic layers, entirely in the HIP
library: prefill (energy, widths, quantize-and-pack), decode attention with its logits, and
bgtq_logit_error against the exact logits of the unquantized keys.  Uniform TQ-MSE is the same
pipeline with every block forced to the same width (b_min = b_max = bits).

    python -m decode_attention_rope_amd.diagnostic [--tokens T] [--layers L] [--time]

prints one JSON line per (panel entry, bits) and a summary line; --time adds the duration of
the logit-error pass on a 128K-token layer with 16 query and 2 KV heads.
"""

from __future__ import annotations

import argparse
import json

import numpy as np
import torch

from . import bgtq, synth

METHODS = ("uniform", "block_gtq")


def layer_inputs(wl: synth.Workload, layer: int, device, capacity: int | None = None):
    """Post-RoPE keys [batch, h_kv, capacity, d] (zero past each length), values, pre-RoPE q."""
    lens = wl.seq_lens
    cap = capacity or max(64, -(-max(lens) // 64) * 64)
    tdt = torch.bfloat16 if wl.key_dtype == "bf16" else torch.float32
    keys = torch.zeros((len(lens), wl.h_kv, cap, wl.d), dtype=tdt, device=device)
    vals = torch.zeros_like(keys)
    for s, t_len in enumerate(lens):
        for h in range(wl.h_kv):
            if t_len:
                keys[s, h, :t_len] = torch.from_numpy(synth.keys(wl, s, layer, h, 0, t_len)).to(device).to(tdt)
                vals[s, h, :t_len] = torch.from_numpy(synth.values(wl, s, layer, h, 0, t_len)).to(device).to(tdt)
    q = torch.from_numpy(np.stack([synth.queries(wl, s, layer) for s in range(len(lens))])).to(device)
    return keys, vals, q, cap


def layer_mae(quantizer, wl: synth.Workload, layer: int, bits: int, method: str, device, inputs=None,
              softmax_scale: float | None = None) -> np.ndarray:
    """Key-only logit MAE per (sequence, query head), fp64 [batch, h_q], for one layer."""
    if method not in METHODS:
        raise ValueError(method)
    keys, vals, q, cap = inputs if inputs is not None else layer_inputs(wl, layer, device)
    n = wl.d // 2
    cache = bgtq.PackedCache(len(wl.seq_lens), wl.h_kv, wl.d, bits * n, bits, cap, device=device)
    b_min, b_max = (bits, bits) if method == "uniform" else (0, 8)
    for s, t_len in enumerate(wl.seq_lens):
        if t_len:
            bgtq.bgtq_prefill(quantizer, cache, keys[s, :, :t_len], vals[s, :, :t_len], s, b_min, b_max)
    _, logits = bgtq.bgtq_decode_attention(quantizer, cache, q, wl.theta, softmax_scale=softmax_scale, logits=True)
    mae = bgtq.bgtq_logit_error(q, keys, cache.lengths, logits, wl.theta, softmax_scale=softmax_scale)
    return mae.cpu().numpy()


def layer_figure(mae: np.ndarray, seq_lens) -> float:
    """Per-layer MAE: mean over heads and tokens (sequences weighted by their token counts)."""
    w = np.asarray(seq_lens, dtype=np.float64)[:, None] * np.ones_like(mae)
    return float(np.sum(mae * w) / np.sum(w)) if np.sum(w) else 0.0


def compare(quantizer, wl: synth.Workload, bits: int, device) -> dict:
    """Per-layer MAE of both methods on every layer of a workload."""
    res = {m: [] for m in METHODS}
    for layer in range(wl.layers):
        inputs = layer_inputs(wl, layer, device)
        for m in METHODS:
            res[m].append(layer_figure(layer_mae(quantizer, wl, layer, bits, m, device, inputs), wl.seq_lens))
    red = [100.0 * (1.0 - g / u) for u, g in zip(res["uniform"], res["block_gtq"])]
    wins = sum(g < u for u, g in zip(res["uniform"], res["block_gtq"]))
    return {"workload": wl.name, "bits": bits, "layers": wl.layers, "tokens": list(wl.seq_lens),
            "mae_uniform": res["uniform"], "mae_block_gtq": res["block_gtq"],
            "reduction_pct": [round(r, 2) for r in red], "wins": f"{wins}/{wl.layers}"}


def time_logit_error(quantizer, device, steps: int = 20) -> dict:
    """Average duration of bgtq_logit_error on one 128K-token layer (16 query, 2 KV heads,
    head_dim 128, fp32 keys) and its HBM roofline fraction."""
    wl = synth.QWEN3B_128K
    keys, vals, q, cap = layer_inputs(wl, 0, device)
    cache = bgtq.PackedCache(1, wl.h_kv, wl.d, wl.budget, wl.v_bits, cap, device=device)
    bgtq.bgtq_prefill(quantizer, cache, keys[0], vals[0], 0)
    _, logits = bgtq.bgtq_decode_attention(quantizer, cache, q, wl.theta, logits=True)
    ws = torch.empty(bgtq.logit_error_workspace_bytes(1, wl.h_q, cap), dtype=torch.uint8, device=device)
    out = torch.empty((1, wl.h_q), dtype=torch.float64, device=device)
    for _ in range(3):
        bgtq.bgtq_logit_error(q, keys, cache.lengths, logits, wl.theta, out=out, workspace=ws)
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        bgtq.bgtq_logit_error(q, keys, cache.lengths, logits, wl.theta, out=out, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * t0.elapsed_time(t1) / steps
    t_len = wl.seq_lens[0]
    # algorithmic bytes: every key once, every logit once, the query heads
    nbytes = wl.h_kv * t_len * wl.d * 4 + wl.h_q * t_len * 4 + wl.h_q * wl.d * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "k_logit_err + k_logit_err_final", "workload": wl.name, "us_per_call": round(us, 2),
            "bytes": nbytes, "achieved_gbs": round(gbs, 1), "peak_gbs": 8000.0, "frac": round(gbs / 8000.0, 4)}


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--bits", type=int, nargs="+", default=[2, 3])
    ap.add_argument("--time", action="store_true")
    ap.add_argument("--time-only", action="store_true", help="skip the panel, time the error pass")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("the diagnostic runs on the GPU (HIP library); no device is visible")
    dev = torch.device("cuda:0")
    quantizers = {}
    wins = total = 0
    reds = []
    for wl in [] if args.time_only else synth.diagnostic_panel(args.tokens, args.layers):
        if wl.d not in quantizers:
            bank = torch.from_numpy(synth.rotation_bank(wl.d)).to(dev)
            rv = torch.from_numpy(synth.rotation_v(wl.d)).to(dev)
            quantizers[wl.d] = (bgtq.make_quantizer(bank, rv, wl.d), bank, rv)
        for bits in args.bits:
            r = compare(quantizers[wl.d][0], wl, bits, dev)
            print(json.dumps(r), flush=True)
            k, n = (int(x) for x in r["wins"].split("/"))
            wins, total = wins + k, total + n
            reds += r["reduction_pct"]
    if reds:
        summary = {"summary": "key-only logit MAE, Block-GTQ vs uniform TQ-MSE", "wins": f"{wins}/{total}",
                   "reduction_pct_min": min(reds), "reduction_pct_median": float(np.median(reds)),
                   "reduction_pct_max": max(reds), "data": "synthetic"}
        print(json.dumps(summary), flush=True)
    if args.time or args.time_only:
        d = synth.QWEN3B_128K.d
        if d not in quantizers:
            bank = torch.from_numpy(synth.rotation_bank(d)).to(dev)
            rv = torch.from_numpy(synth.rotation_v(d)).to(dev)
            quantizers[d] = (bgtq.make_quantizer(bank, rv, d), bank, rv)
        print(json.dumps(time_logit_error(quantizers[d][0], dev)), flush=True)


if __name__ == "__main__":
    main()
