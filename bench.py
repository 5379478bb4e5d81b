"""Decode throughput of the Block-GTQ packed-cache path on one MI355X.

Workloads (--workload; synthetic inputs shaped like the pages' models, resident in HBM before
timing starts):
  qwen3b_36L_128k_K3V3      (default) Qwen2.5-3B shape: 16 query / 2 KV heads, head_dim 128,
                            rope_theta 1e6, 36 layers in sequence, batch 1, 131072 cached
                            tokens, K3V3.
  qwen3b_36L_512k_K3V3      the same at 524288 cached tokens (packed footprint reported against
                            the fp16 one).
  llama8b_layer_32k_K2V2    Llama-3.1-8B-shaped single layer (32 / 8 heads), 32K tokens, bf16
                            keys, K2V2; 32 copies of the cache are stepped in turn so that the
                            reads come from HBM, not from the 256 MB last-level cache.
  qwen7b_28L_ragged16_K3V2  7B-Qwen shape (28 / 4 heads, 28 layers), batch of 16 sequences with
                            seeded lengths in [8K, 64K], K3V2; also times a fresh 32K-token
                            prefill (energy, allocation, quantize-and-append) of 16 sequences.
  tiny_d64_T256_K3V3        the tiny single-head case.

One step = for every layer: quantize-and-append one new token per sequence, then decode
attention over the whole cache (bgtq_decode_step, append-then-attend).  The step is captured
once in a HIP graph and replayed.  Prints one JSON line: throughput (decode tokens/s), the
roofline of the decode call (HBM bound), and the CPU oracle timed on a bounded sample of the
same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "decode_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_rope_amd", "csrc", f) for f in ("kernels.hip", "decode_stream.h")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="qwen3b_36L_128k_K3V3")
    p.add_argument("--kernel-reps", type=int, default=20, help="graph replays for the decode-call timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="timed oracle seconds per CPU figure")
    p.add_argument("--rotation", choices=("dense", "givens"), default="dense",
                   help="TQ-MSE rotation kind: dense Haar matrices (default) or structured Givens layers")
    p.add_argument("--window", type=int, default=0,
                   help="fp16 recent-key window in tokens (0: none, the default workload)")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="after timing, run one plain device copy of this many MiB (scale for PMC byte counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload(name):
    from decode_attention_rope_amd import synth
    table = {w.name: w for w in (synth.TINY, synth.LLAMA8B_LAYER, synth.QWEN3B_128K, synth.QWEN3B_512K,
                                 synth.QWEN7B_RAGGED)}
    if name not in table:
        raise SystemExit(f"unknown workload {name!r}; one of {sorted(table)}")
    return table[name]


def copies_of(wl) -> int:
    """Distinct caches stepped in turn per layer: enough that a single-layer workload's reads come
    from HBM (26 x 20 MB already exceed the 256 MB last-level cache)."""
    return 32 if wl.layers == 1 and wl.name.startswith("llama") else 1


def bytes_per_token_head(widths_row, v_bits, d) -> int:
    """Algorithmic bytes one cached token of one KV head costs a decode: codes and fp16 norms."""
    w = [int(x) for x in widths_row]
    k_code_bits = 2 * sum(w)
    groups = len({x for x in w if x > 0})
    return k_code_bits // 8 + 2 * groups + v_bits * d // 8 + 2


def kernel_source_hash(texts=None) -> str:
    """sha256 of the decode kernels' sources with comments and blank space removed, so that a
    comment edit does not invalidate counters taken on the same code."""
    import re
    h = hashlib.sha256()
    if texts is None:
        texts = []
        for p in KERNEL_SOURCES:
            with open(p) as f:
                texts.append(f.read())
    for t in texts:
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
    return h.hexdigest()


def stored_counters(workload_name: str):
    """The rocprofv3 PMC figures stored for this workload (profiles/decode_counters.json), if they
    were taken on the current kernel sources; None otherwise."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except OSError:
        return None
    entry = rec.get("workloads", {}).get(workload_name)
    if not entry or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return entry


# ------------------------------------------------------------------ CPU baseline (the oracle)

def _cpu_facts() -> dict:
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    quota = None                              # the cgroup's CPU time limit, in cores
    for path in ("/sys/fs/cgroup/cpu.max", "/sys/fs/cgroup/cpu/cpu.cfs_quota_us"):
        try:
            with open(path) as f:
                parts = f.read().split()
        except OSError:
            continue
        if path.endswith("cpu.max") and parts and parts[0] != "max":
            quota = int(parts[0]) / int(parts[1])
        elif path.endswith("quota_us") and parts and int(parts[0]) > 0:
            with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
                quota = int(parts[0]) / int(f.read().split()[0])
        break
    return {"affinity_cores": cores, "cgroup_cpu_quota_cores": quota, "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _oracle_units(wl):
    """(layer, seq, kv head) units of one decode step, and the sample the baseline runs: all KV
    heads of the first layer (first two sequences of a batch)."""
    n_seq = min(len(wl.seq_lens), 2)
    return [(0, s, h) for s in range(n_seq) for h in range(wl.h_kv)]


def _oracle_prepare(wl_name, unit):
    """Untimed set-up of one unit: the oracle's quantized cache of it (prefill by the oracle's
    energy, allocation and quantizer, then the new token quantized with that allocation)."""
    from decode_attention_rope_amd import synth
    from oracle import allocate, energy, layout, quantize
    wl = workload(wl_name)
    layer, s, h = unit
    t_len = wl.seq_lens[s] + 1
    bank, rv = synth.rotation_bank(wl.d), synth.rotation_v(wl.d)
    k = synth.keys(wl, s, layer, h, 0, t_len)
    v = synth.values(wl, s, layer, h, 0, t_len)
    lay = layout.build(allocate.greedy(energy.block_energy(k[:-1]), wl.budget))
    kc, kn = quantize.quantize_keys(k, lay, bank)
    vc, vn = quantize.quantize_values(v, rv, wl.v_bits)
    q = synth.queries(wl, s, layer)[h * wl.group:(h + 1) * wl.group]
    return (wl, lay, kc, kn, vc, vn, q, t_len, bank, rv)


def _oracle_decode(prep):
    """The timed unit: dequantize the unit's keys and values, fp64 attention of its query group."""
    from oracle import decode, quantize
    wl, lay, kc, kn, vc, vn, q, t_len, bank, rv = prep
    kh = quantize.dequantize_keys(kc, kn, lay, bank)
    vh = quantize.dequantize_values(vc, vn, rv, wl.v_bits)
    decode.decode_head_group(q, t_len - 1, wl.theta, kh, vh)


def _oracle_worker(wl_name, unit, seconds, barrier, results):
    import numpy  # noqa: F401  (the BLAS libraries must be loaded before they are limited)
    from threadpoolctl import threadpool_limits
    from oracle import allocate, decode, energy, layout, quantize  # noqa: F401
    with threadpool_limits(1):
        prep = _oracle_prepare(wl_name, unit)
        barrier.wait()
        reps, t0 = 0, time.perf_counter()
        while True:
            _oracle_decode(prep)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
    results.put((reps, dt))


def cpu_baseline(wl, seconds: float):
    """The oracle as it stands, timed on the host cores: one process with one BLAS thread, then N
    processes (N = the cores this process may run on, at most 16 and at most the cgroup's CPU
    quota) with one BLAS thread each,
    every process decoding one (layer, sequence, KV head) unit of the sample again and again for
    `seconds`.  Throughput is extrapolated to whole decode steps (units per step / units per
    second).  `value` is the better of the two figures, `cores` the processes it used."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits

    facts = _cpu_facts()
    units = _oracle_units(wl)
    per_step = wl.layers * len(wl.seq_lens) * wl.h_kv       # units in one decode step
    batch = len(wl.seq_lens)
    # one process, one BLAS thread, the units in turn
    with threadpool_limits(1):
        preps = [_oracle_prepare(wl.name, u) for u in units]
        reps, t0 = 0, time.perf_counter()
        while True:
            _oracle_decode(preps[reps % len(preps)])
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
    del preps
    single = batch * (reps / dt) / per_step
    # N processes: the cores this process may use, at most 16 and at most the cgroup's CPU quota
    n_proc = min(16, facts["affinity_cores"])
    if facts["cgroup_cpu_quota_cores"]:
        n_proc = min(n_proc, int(facts["cgroup_cpu_quota_cores"]))
    n_proc = max(1, n_proc)
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(n_proc), ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(wl.name, units[i % len(units)], seconds, barrier, results))
             for i in range(n_proc)]
    for p in procs:
        p.start()
    got = [results.get(timeout=seconds * 4 + 600) for _ in procs]
    for p in procs:
        p.join()
    multi = batch * sum(r / t for r, t in got) / per_step
    best, best_cores = (multi, n_proc) if multi >= single else (single, 1)
    return {"value": best, "unit": "tok/s", "cores": best_cores, "kind": "oracle",
            "single_process": {"value": single, "unit": "tok/s", "cores": 1},
            "n_processes": {"value": multi, "unit": "tok/s", "cores": n_proc},
            **facts,
            "sample": (f"the oracle decodes one (layer, sequence, KV head) unit at a time: dequantize the "
                       f"packed keys and values and fp64 attention of the unit's {wl.group} query heads; units "
                       f"are the {len(units)} (sequence, KV head) pairs of layer 0"
                       f"{' (first 2 sequences)' if batch > 2 else ''} at their full lengths; each figure "
                       f"runs {seconds:g} s; tok/s = batch x units per second / {per_step} units per "
                       f"decode step; one BLAS thread per process")}


# ------------------------------------------------------------------ GPU run

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path is single-GPU.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from decode_attention_rope_amd import bgtq, synth

    wl = workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bgtq.init()
    batch = len(wl.seq_lens)
    n_copy = copies_of(wl)
    steps_total = args.warmup + args.steps + 2
    # a step appends one token to every cache it touches; with n_copy copies each copy takes
    # one step in n_copy
    cap = -(-(max(wl.seq_lens) + steps_total) // 64) * 64
    if args.rotation == "givens":
        giv = torch.from_numpy(synth.givens_bank(wl.d).view(np.int32)).to(dev)
        qz = bgtq.make_quantizer(None, None, wl.d, givens=giv)
    else:
        bank = torch.from_numpy(synth.rotation_bank(wl.d)).to(dev)
        rv = torch.from_numpy(synth.rotation_v(wl.d)).to(dev)
        qz = bgtq.make_quantizer(bank, rv, wl.d)

    # ---------------- prefill every layer (set-up, not in the metric)
    log(f"prefill {wl.layers} layers x {batch} sequences x {wl.h_kv} KV heads ({n_copy} copies)")
    caches, layer_of = [], []
    pre_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    pre_ms = 0.0
    for layer in range(wl.layers):
        cache = bgtq.PackedCache(batch, wl.h_kv, wl.d, wl.budget, wl.v_bits, cap, device=dev, window=args.window)
        for s, t_len in enumerate(wl.seq_lens):
            kv = [synth.keys_values_device(wl, s, layer, h, t_len, dev) for h in range(wl.h_kv)]
            k = torch.stack([x[0] for x in kv]).contiguous()
            v = torch.stack([x[1] for x in kv]).contiguous()
            del kv
            pre_ev[0].record()
            bgtq.bgtq_prefill(qz, cache, k, v, s)
            pre_ev[1].record()
            torch.cuda.synchronize()
            pre_ms += pre_ev[0].elapsed_time(pre_ev[1])
            del k, v
        assert int(cache.status[0]) == 0
        caches.append(cache)
        layer_of.append(layer)
        for _ in range(n_copy - 1):          # the same bytes at other addresses
            c2 = bgtq.PackedCache(batch, wl.h_kv, wl.d, wl.budget, wl.v_bits, cap, device=dev, window=args.window)
            for name in ("k_codes", "k_norms", "v_codes", "v_norms", "lengths", "widths", "layouts", "status"):
                getattr(c2, name).copy_(getattr(cache, name))
            if cache.k_window is not None:
                c2.k_window.copy_(cache.k_window)
            caches.append(c2)
            layer_of.append(layer)
    torch.cuda.synchronize()
    n_cache = len(caches)

    # ---------------- per-cache decode inputs (fixed, resident)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    q_layer = [torch.from_numpy(np.stack([synth.queries(wl, s, layer) for s in range(batch)])).to(dev)
               for layer in range(wl.layers)]
    k_new = [torch.randn((batch, wl.h_kv, 1, wl.d), generator=gen, device=dev) for _ in range(n_cache)]
    v_new = [torch.randn((batch, wl.h_kv, 1, wl.d), generator=gen, device=dev) for _ in range(n_cache)]
    outs = [torch.empty((batch, wl.h_q, wl.d), device=dev) for _ in range(n_cache)]
    ws_bytes = bgtq.decode_workspace_bytes(batch, wl.h_q, wl.h_kv, wl.d, cap)
    wss = [torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_cache)]

    def steps_of_graph():
        """One graph = n_copy decode steps: each copy of every layer exactly once."""
        for i in range(n_cache):
            bgtq.bgtq_decode_step(qz, caches[i], q_layer[layer_of[i]], k_new[i], v_new[i], wl.theta,
                                  out=outs[i], workspace=wss[i])

    def decode_calls():
        for i in range(n_cache):
            bgtq.bgtq_decode_attention(qz, caches[i], q_layer[layer_of[i]], wl.theta, out=outs[i], workspace=wss[i])

    # ---------------- capture the step(s) in a HIP graph (the first real step runs eagerly)
    steps_of_graph()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps_of_graph()
    torch.cuda.synchronize()
    for _ in range(max(args.warmup - 1, 0)):
        graph.replay()
    torch.cuda.synchronize()
    replays = max(1, -(-args.steps // n_copy))
    log(f"timing {replays * n_copy} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    steps_timed = replays * n_copy
    ms_per_step = e0.elapsed_time(e1) / steps_timed
    lengths = [c.lengths.cpu().tolist() for c in caches]
    assert all(int(c.status[0]) == 0 for c in caches)
    assert all(torch.isfinite(o).all() for o in outs)

    # ---------------- the decode call: HIP events around graph replays of one call per cache
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        decode_calls()
    dgraph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.kernel_reps):
        dgraph.replay()
    e1.record()
    torch.cuda.synchronize()
    us_per_call = e0.elapsed_time(e1) * 1e3 / (args.kernel_reps * n_cache)
    # algorithmic bytes of one call: every cached token's packed codes and fp16 norms, per
    # (sequence, KV head) at its own widths; tokens in the window as fp16 keys plus their values
    call_bytes = []
    for i, c in enumerate(caches):
        w = c.widths.cpu().numpy()
        tot = 0.0
        for s in range(batch):
            t = lengths[i][s]
            n_win = min(args.window, t)
            for h in range(wl.h_kv):
                tot += bytes_per_token_head(w[s, h], wl.v_bits, wl.d) * (t - n_win)
                tot += n_win * (2 * wl.d + wl.v_bits * wl.d // 8 + 2)
        call_bytes.append(tot)
    bytes_per_call = float(np.mean(call_bytes))
    achieved = bytes_per_call / (us_per_call * 1e-6) / 1e9
    packed_bytes_layer = caches[0].nbytes
    ctx = max(max(l) for l in lengths)

    extra = {}
    if wl.name.startswith("qwen7b"):
        extra["prefill_32k"] = time_fresh_prefill(wl, qz, dev)
    if wl.name.startswith("qwen3b"):
        t = wl.seq_lens[0]
        fp16 = wl.h_kv * wl.d * 2 * 2 * wl.layers * t
        packed = packed_bytes_layer * wl.layers
        extra["footprint"] = {"packed_cache_gb": packed / 1e9, "fp16_cache_gb": fp16 / 1e9,
                              "ratio": fp16 / packed,
                              "note": "packed = codes and fp16 norms of every layer at capacity "
                                      f"{cap}; fp16 = 2 KV heads x head_dim x 2 bytes x (K, V) x layers x {t}"}

    if args.copy_mb > 0:   # a plain copy kernel of known size, for counter calibration
        src = torch.ones(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    counters = stored_counters(wl.name) if args.window == 0 and args.rotation == "dense" else None
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": counters["traffic_bytes_per_call"] if counters else None,
                "kernel": "one bgtq_decode_attention call (k_decode_stream split pass + k_decode_combine), "
                          "timed per call with HIP events around graph replays",
                "us_per_call": us_per_call, "alg_bytes_per_call": bytes_per_call}
    if counters:
        roofline["traffic_source"] = f"stored rocprofv3 PMC of these kernel sources ({counters['summary']})"
        roofline["valu_busy_frac"] = counters.get("valu_busy_frac")
    result = {
        "metric": "decode-attn tok/s + achieved HBM GB/s (% peak), packed K3V3 cache, 128K ctx",
        "value": batch * 1000.0 / ms_per_step,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp16 MFMA operands (key levels and query as fp16 hi+lo pairs, value levels "
                  + ("as hi+lo pairs" if args.window else "as fp16") + "), fp32 accumulation"),
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "q_heads": wl.h_q, "kv_heads": wl.h_kv,
                   "head_dim": wl.d, "context": ctx, "batch": batch, "budget": f"K{wl.k_bits}V{wl.v_bits}",
                   "capacity": cap, "recent_key_window": args.window, "rotation": args.rotation,
                   "cache_copies": n_copy},
        "roofline": roofline,
        "prefill_ms_per_layer": pre_ms / wl.layers,
        "packed_cache_bytes_per_layer": packed_bytes_layer,
        **extra,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result))


def time_fresh_prefill(wl, qz, dev, t_len: int = 32768):
    """Energy + allocation + quantize-and-append (bgtq_prefill) of a fresh t_len-token prefix of
    every sequence of the batch, one layer, timed with HIP events (keys generated beforehand)."""
    import torch
    from decode_attention_rope_amd import bgtq, synth
    batch = len(wl.seq_lens)
    cache = bgtq.PackedCache(batch, wl.h_kv, wl.d, wl.budget, wl.v_bits, -(-t_len // 64) * 64, device=dev)
    kvs = []
    for s in range(batch):
        kv = [synth.keys_values_device(wl, s, 0, h, t_len, dev) for h in range(wl.h_kv)]
        kvs.append((torch.stack([x[0] for x in kv]).contiguous(), torch.stack([x[1] for x in kv]).contiguous()))
    ws = torch.empty(max(int(bgtq.lib().bgtq_prefill_workspace_bytes(wl.h_kv, t_len, wl.d)), 8), dtype=torch.uint8,
                     device=dev)
    for s in range(batch):          # once untimed (first-use costs)
        bgtq.bgtq_prefill(qz, cache, kvs[s][0], kvs[s][1], s, workspace=ws)
    cache.lengths.zero_()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(batch):
        bgtq.bgtq_prefill(qz, cache, kvs[s][0], kvs[s][1], s, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert int(cache.status[0]) == 0
    return {"ms_per_layer": ms, "tokens": batch * t_len, "sequences": batch, "kv_heads": wl.h_kv,
            "tokens_per_s": batch * t_len / (ms * 1e-3),
            "ms_all_layers": ms * wl.layers, "what": "bgtq_prefill (energy, allocation, quantize-and-append) "
                                                   f"of {batch} sequences x {t_len} tokens x {wl.h_kv} KV heads"}


if __name__ == "__main__":
    main()
