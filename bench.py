"""Decode throughput of the Block-GTQ packed-cache path on one MI355X.

Workload (default): Qwen2.5-3B-shaped decode -- 16 query heads, 2 KV heads,
head_dim 128, rope_theta 1e6, 36 layers run in sequence, batch 1, 131072
cached tokens, K3V3 budget.  One step = for every layer: quantize-and-append
the new token's key and value, then decode attention over the whole cache
(append-then-attend).  The 36-layer step is captured once in a HIP graph and
replayed; inputs are synthetic and resident in HBM before timing starts.

Prints one JSON line with the throughput (decode tokens/s), the roofline of
the dominant kernel (decode attention, HBM bound) and the CPU oracle timed on
a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="qwen3b_36L_128k_K3V3")
    p.add_argument("--kernel-reps", type=int, default=20, help="graph replays for the kernel timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--rotation", choices=("dense", "givens"), default="dense",
                   help="TQ-MSE rotation kind: dense Haar matrices (default) or structured Givens layers")
    p.add_argument("--window", type=int, default=0,
                   help="fp16 recent-key window in tokens (0: none, the default workload)")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="after timing, run one plain device copy of this many MiB (scale for PMC byte counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bytes_per_token_head(widths_row, v_bits, d) -> int:
    """Algorithmic bytes one cached token of one KV head costs a decode: codes and fp16 norms."""
    w = [int(x) for x in widths_row]
    k_code_bits = 2 * sum(w)
    groups = len({x for x in w if x > 0})
    return k_code_bits // 8 + 2 * groups + v_bits * d // 8 + 2


def measured_traffic(workload: str):
    """HBM bytes of one decode call from the committed rocprofv3 byte counters (profiles/), or None
    when they were taken on another workload or on a kernel source that has changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    src = os.path.join(ROOT, "decode_attention_rope_amd", "csrc", "kernels.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != sha or rec.get("workload") != workload:
        return None
    return float(rec["traffic_bytes_per_call"])


def cpu_baseline(wl, layer_sample: int = 1, min_seconds: float = 10.0):
    """The oracle, as it stands, on `layer_sample` of the workload's layers (one decode step each),
    the timed decode repeated until it has run for at least `min_seconds`."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from decode_attention_rope_amd import synth
    from oracle import allocate, decode, energy, layout, quantize

    t_len = wl.seq_lens[0] + 1
    bank, rv = synth.rotation_bank(wl.d), synth.rotation_v(wl.d)
    heads = []
    for layer in range(layer_sample):
        for h in range(wl.h_kv):
            k = synth.keys(wl, 0, layer, h, 0, t_len)
            v = synth.values(wl, 0, layer, h, 0, t_len)
            lay = layout.build(allocate.greedy(energy.block_energy(k[:-1]), wl.budget))
            kc, kn = quantize.quantize_keys(k, lay, bank)
            vc, vn = quantize.quantize_values(v, rv, wl.v_bits)
            heads.append((layer, h, lay, kc, kn, vc, vn))
    q = {layer: synth.queries(wl, 0, layer) for layer in range(layer_sample)}
    reps, t0 = 0, time.perf_counter()
    while True:
        for layer, h, lay, kc, kn, vc, vn in heads:
            kh = quantize.dequantize_keys(kc, kn, lay, bank)
            vh = quantize.dequantize_values(vc, vn, rv, wl.v_bits)
            decode.decode_head_group(q[layer][h * wl.group:(h + 1) * wl.group], t_len - 1, wl.theta, kh, vh)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 100:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    per_step = dt / reps * wl.layers / layer_sample
    return {"value": 1.0 / per_step, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one decode step of {layer_sample} of {wl.layers} layers (all {wl.h_kv} KV heads x "
                      f"{t_len} tokens, dequantize + fp64 attention), run {reps} times in {dt:.1f} s, "
                      f"extrapolated x{wl.layers / layer_sample:g}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path is single-GPU.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from decode_attention_rope_amd import bgtq, synth

    wl = synth.WORKLOADS[args.workload]
    assert len(wl.seq_lens) == 1, "bench times a batch-1 workload"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bgtq.init()
    t_len = wl.seq_lens[0]
    steps_total = args.warmup + args.steps + 1
    cap = -(-(t_len + steps_total) // 64) * 64
    if args.rotation == "givens":
        giv = torch.from_numpy(synth.givens_bank(wl.d).view(np.int32)).to(dev)
        qz = bgtq.make_quantizer(None, None, wl.d, givens=giv)
    else:
        bank = torch.from_numpy(synth.rotation_bank(wl.d)).to(dev)
        rv = torch.from_numpy(synth.rotation_v(wl.d)).to(dev)
        qz = bgtq.make_quantizer(bank, rv, wl.d)

    # ---------------- prefill every layer (setup, not timed in the metric)
    log(f"prefill {wl.layers} layers x {wl.h_kv} KV heads x {t_len} tokens")
    caches, layer_bytes = [], []
    pre_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    pre_ms = 0.0
    for layer in range(wl.layers):
        cache = bgtq.PackedCache(1, wl.h_kv, wl.d, wl.budget, wl.v_bits, cap, device=dev, window=args.window)
        kv = [synth.keys_values_device(wl, 0, layer, h, t_len, dev) for h in range(wl.h_kv)]
        k = torch.stack([x[0] for x in kv]).contiguous()
        v = torch.stack([x[1] for x in kv]).contiguous()
        del kv
        pre_ev[0].record()
        bgtq.bgtq_prefill(qz, cache, k, v, 0)
        pre_ev[1].record()
        torch.cuda.synchronize()
        pre_ms += pre_ev[0].elapsed_time(pre_ev[1])
        del k, v
        caches.append(cache)
        w = cache.widths.cpu().numpy()[0]
        layer_bytes.append([bytes_per_token_head(w[h], wl.v_bits, wl.d) for h in range(wl.h_kv)])
    torch.cuda.synchronize()
    assert all(int(c.status[0]) == 0 for c in caches)

    # ---------------- per-layer decode inputs (fixed, resident)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    qs = [torch.from_numpy(synth.queries(wl, 0, layer)[None]).to(dev) for layer in range(wl.layers)]
    k_new = [torch.randn((1, wl.h_kv, 1, wl.d), generator=gen, device=dev) for _ in range(wl.layers)]
    v_new = [torch.randn((1, wl.h_kv, 1, wl.d), generator=gen, device=dev) for _ in range(wl.layers)]
    outs = [torch.empty((1, wl.h_q, wl.d), device=dev) for _ in range(wl.layers)]
    ws_bytes = bgtq.decode_workspace_bytes(1, wl.h_q, wl.h_kv, wl.d, cap)
    wss = [torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(wl.layers)]

    def step():
        for layer in range(wl.layers):
            bgtq.bgtq_decode_step(qz, caches[layer], qs[layer], k_new[layer], v_new[layer], wl.theta,
                                  out=outs[layer], workspace=wss[layer])

    def decode_only():
        for layer in range(wl.layers):
            bgtq.bgtq_decode_attention(qz, caches[layer], qs[layer], wl.theta, out=outs[layer],
                                       workspace=wss[layer])

    # ---------------- capture the 36-layer step in a HIP graph (first real step runs eagerly)
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup - 1 if args.warmup > 0 else 0):
        graph.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    lengths = [int(c.lengths[0]) for c in caches]
    assert len(set(lengths)) == 1 and all(int(c.status[0]) == 0 for c in caches)
    assert all(torch.isfinite(o).all() for o in outs)

    # ---------------- dominant kernel: decode attention, timed with events around graph replays
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        decode_only()
    dgraph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.kernel_reps):
        dgraph.replay()
    e1.record()
    torch.cuda.synchronize()
    us_per_launch = e0.elapsed_time(e1) * 1e3 / (args.kernel_reps * wl.layers)
    ctx = lengths[0]
    # tokens in the window are read as fp16 keys plus their packed values and value norms
    n_win = min(args.window, ctx)
    win_bytes = wl.h_kv * n_win * (2 * wl.d + wl.v_bits * wl.d // 8 + 2)
    bytes_per_launch = float(np.mean([sum(b) for b in layer_bytes])) * (ctx - n_win) + win_bytes
    achieved = bytes_per_launch / (us_per_launch * 1e-6) / 1e9

    if args.copy_mb > 0:   # a plain copy kernel of known size, for counter calibration
        src = torch.ones(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    result = {
        "metric": "decode-attn tok/s + achieved HBM GB/s (% peak), packed K3V3 cache, 128K ctx",
        "value": 1000.0 / ms_per_step,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "q_heads": wl.h_q, "kv_heads": wl.h_kv,
                   "head_dim": wl.d, "context": ctx, "batch": 1, "budget": f"K{wl.k_bits}V{wl.v_bits}",
                   "capacity": cap, "recent_key_window": args.window, "rotation": args.rotation},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wl.name) if args.window == 0 and args.rotation == "dense" else None,
                     "kernel": "decode attention: one bgtq_decode_attention call per layer "
                               "(k_decode_mfma + k_decode_combine)",
                     "us_per_launch": us_per_launch, "alg_bytes_per_launch": bytes_per_launch},
        "prefill_ms_per_layer": pre_ms / wl.layers,
        "packed_cache_bytes_per_layer": caches[0].nbytes,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
