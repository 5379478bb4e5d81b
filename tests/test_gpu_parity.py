"""GPU parity: the HIP path through the C ABI against the CPU oracle (needs an MI355X).

Bit-exact: energies, widths, layout descriptors, codes, norms and packed bytes.
Within 2e-3 normwise max relative error per (sequence, query head): logits and outputs.
"""

import numpy as np
import pytest
import torch

from decode_attention_rope_amd import bgtq, synth
from oracle import allocate, codebook, energy, layout, rope
from _ref import TOL, assert_region_equal, decode_reference, head_reference, oracle_heads, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device(DEV)


def _t(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def rot128():
    _cuda()
    bank, rv = synth.rotation_bank(128), synth.rotation_v(128)
    return bank, rv, bgtq.make_quantizer(_t(bank), _t(rv), 128)


@pytest.fixture(scope="module")
def rot64():
    _cuda()
    bank, rv = synth.rotation_bank(64), synth.rotation_v(64)
    return bank, rv, bgtq.make_quantizer(_t(bank), _t(rv), 64)


# ---------------------------------------------------------------- energy

@pytest.mark.parametrize("t_len,dtype,pairing", [(1, "f32", 0), (255, "f32", 1), (256, "bf16", 0),
                                                 (257, "f32", 0), (5000, "bf16", 1), (70000, "f32", 0)])
def test_block_energy_bit_exact(t_len, dtype, pairing):
    _cuda()
    _say(f"energy T={t_len} {dtype} pairing={pairing}")
    rng = np.random.default_rng(t_len)
    k = (rng.standard_normal((3, t_len, 128)) * np.exp(rng.uniform(-3, 2, size=(3, 1, 128)))).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kt = _t(k, tdt)
    k_exact = kt.float().cpu().numpy()
    # a strided view: heads interleaved with padding
    big = torch.zeros((3, t_len, 160), dtype=tdt, device=DEV)
    big[:, :, :128] = kt
    got = bgtq.bgtq_block_energy(big[:, :, :128], pairing).cpu().numpy()
    want = np.stack([energy.block_energy(k_exact[h], pairing) for h in range(3)])
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- allocation

def _layout_fields(raw: np.ndarray):
    i32 = raw[:144].view(np.int32)
    return {"n_groups": i32[0], "d_eff": i32[1], "code_bits": i32[2], "chunks": i32[3],
            "g_width": i32[4:12], "g_first": i32[12:20], "g_m": i32[20:28], "g_bitoff": i32[28:36],
            "perm": raw[144:400], "group": raw[400:656], "offset": raw[656:1168].view(np.uint16)}


@pytest.mark.parametrize("n,seed", [(32, 0), (64, 1), (64, 2), (128, 3)])
def test_allocate_bit_exact(n, seed):
    _cuda()
    _say(f"allocate n={n} seed={seed}")
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(12):
        kind = i % 4
        e = [rng.exponential(size=n), np.exp(rng.uniform(-9, 1, size=n)),
             rng.integers(0, 3, size=n).astype(float), np.full(n, 0.5)][kind]
        b_min = int(rng.integers(0, 3))
        b_max = int(rng.integers(max(b_min, 1), 9))
        budget = int(rng.integers(n * b_min, n * b_max + 1))
        cases.append((e, budget, b_min, b_max, int(rng.integers(2))))
    for e, budget, b_min, b_max, pairing in cases:
        w, lay = bgtq.bgtq_allocate_bits(_t(e[None], torch.float64), budget, b_min, b_max, pairing)
        want = allocate.greedy(e, budget, b_min, b_max)
        np.testing.assert_array_equal(w.cpu().numpy()[0], want)
        ref = layout.build(want, pairing)
        f = _layout_fields(lay.cpu().numpy()[0])
        assert f["n_groups"] == len(ref.groups) and f["d_eff"] == ref.d_eff
        assert f["code_bits"] == ref.code_bits and f["chunks"] == ref.chunks
        for g, grp in enumerate(ref.groups):
            assert (f["g_width"][g], f["g_first"][g], f["g_m"][g], f["g_bitoff"][g]) == \
                (grp.width, grp.first, grp.m, grp.bit_offset)
        np.testing.assert_array_equal(f["perm"][:ref.d_eff], ref.perm)
        np.testing.assert_array_equal(f["offset"][:ref.d_eff], ref.offset)


# ---------------------------------------------------------------- quantize + pack

@pytest.mark.parametrize("d,k_bits,v_bits,appends", [
    (128, 3, 3, [100, 1, 37, 64, 5]),
    (128, 2, 2, [300]),
    (64, 3, 1, [1, 1, 70, 33]),
    (128, 8, 8, [65]),
    (128, 0, 3, [40]),
    (256, 3, 2, [129]),
    (72, 3, 3, [100, 1, 37, 5]),      # head dims that are not multiples of 16 or 64
    (200, 3, 2, [70, 1, 33]),
])
def test_quantize_append_bytes_bit_exact(d, k_bits, v_bits, appends):
    dev = _cuda()
    _say(f"append d={d} K{k_bits}V{v_bits} appends={appends}")
    t_len = sum(appends)
    cap = -(-t_len // 64) * 64 + 64
    wl = synth.Workload("append_case", 90, d=d, h_q=4, h_kv=2, theta=1e4, layers=1, seq_lens=(t_len,),
                        k_bits=k_bits, v_bits=v_bits, key_dtype="f32", profile="decay", outlier_blocks=2)
    bank, rv = synth.rotation_bank(d, seed=5), synth.rotation_v(d, seed=5)
    qz = bgtq.make_quantizer(_t(bank), _t(rv), d)
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
        ref = head_reference(k[h], v[h], wl.budget, v_bits, bank, rv, cap)
        np.testing.assert_array_equal(cache.widths[0, h].cpu().numpy(), ref["widths"])
        assert_region_equal(cache.region(0, h), ref["region"], t_len, ref["layout"], v_bits, d)


def test_capacity_overflow_sets_status(rot64):
    dev = _cuda()
    bank, rv, qz = rot64
    cache = bgtq.PackedCache(2, 1, 64, 96, 3, 128, device=dev)
    k = torch.randn((2, 1, 100, 64), device=dev)
    e = bgtq.bgtq_block_energy(k[0])
    for s in range(2):
        bgtq.bgtq_allocate_bits(e, 96, widths_out=cache.widths[s], layouts_out=cache.layouts[s])
    bgtq.bgtq_quantize_append(qz, cache, k, k)
    before = cache.k_codes.clone()
    bgtq.bgtq_quantize_append(qz, cache, k[:, :, :50].contiguous(), k[:, :, :50].contiguous())
    torch.cuda.synchronize()
    assert cache.lengths.tolist() == [100, 100]
    assert int(cache.status[0]) == 1
    assert torch.equal(before, cache.k_codes)


@pytest.mark.parametrize("d,k_bits,v_bits,h_kv,prefill,steps,dtype,seq_begin", [
    (128, 3, 3, 2, [60, 0, 130], 70, "f32", 0),     # three sequences, tile crossings
    (64, 2, 5, 6, [10, 63], 40, "bf16", 0),         # more heads than one pass, straddling value codes
    (64, 3, 3, 3, [7, 20], 30, "f32", 1),           # only the second sequence grows
    (256, 3, 7, 1, [5], 70, "f32", 0),
    (128, 0, 3, 2, [3], 66, "f32", 0),              # zero key budget
    (72, 3, 3, 2, [60, 5], 40, "f32", 0),           # head dims that are not multiples of 16
    (200, 2, 3, 1, [10], 30, "bf16", 0),
])
def test_append_one_token_per_step_bit_exact(d, k_bits, v_bits, h_kv, prefill, steps, dtype, seq_begin):
    """Decode-style appends (one token per sequence per call) against the oracle, byte for byte."""
    dev = _cuda()
    _say(f"append-one d={d} K{k_bits}V{v_bits} h_kv={h_kv} prefill={prefill} steps={steps} {dtype} sb={seq_begin}")
    n_seq = len(prefill)
    grow = list(range(seq_begin, n_seq))
    t_lens = [p + (steps if s in grow else 0) for s, p in enumerate(prefill)]
    cap = -(-max(t_lens) // 64) * 64 + 64
    wl = synth.Workload("append_one", 91, d=d, h_q=h_kv, h_kv=h_kv, theta=1e4, layers=1, seq_lens=tuple(t_lens),
                        k_bits=k_bits, v_bits=v_bits, key_dtype=dtype, profile="decay", outlier_blocks=2)
    bank, rv = synth.rotation_bank(d, seed=7), synth.rotation_v(d, seed=7)
    qz = bgtq.make_quantizer(_t(bank), _t(rv), d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ks = [np.stack([synth.keys(wl, s, 0, h, 0, t_lens[s]) for h in range(h_kv)]) for s in range(n_seq)]
    vs = [np.stack([synth.values(wl, s, 0, h, 0, t_lens[s]) for h in range(h_kv)]) for s in range(n_seq)]
    cache = bgtq.PackedCache(n_seq, h_kv, d, wl.budget, v_bits, cap, device=dev)
    for s in range(n_seq):
        bgtq.bgtq_allocate_bits(bgtq.bgtq_block_energy(_t(ks[s])), wl.budget, widths_out=cache.widths[s],
                                layouts_out=cache.layouts[s])
        if prefill[s]:
            bgtq.bgtq_quantize_append(qz, cache, _t(ks[s][:, :prefill[s]])[None].to(tdt),
                                      _t(vs[s][:, :prefill[s]])[None].to(tdt), seq_begin=s)
    for step in range(steps):
        kn = torch.stack([_t(ks[s][:, prefill[s] + step:prefill[s] + step + 1]) for s in grow]).to(tdt)
        vn = torch.stack([_t(vs[s][:, prefill[s] + step:prefill[s] + step + 1]) for s in grow]).to(tdt)
        bgtq.bgtq_quantize_append(qz, cache, kn.contiguous(), vn.contiguous(), seq_begin=seq_begin)
    torch.cuda.synchronize()
    assert cache.lengths.tolist() == t_lens and int(cache.status[0]) == 0
    for s in range(n_seq):
        for h in range(h_kv):
            ref = head_reference(ks[s][h], vs[s][h], wl.budget, v_bits, bank, rv, cap)
            assert_region_equal(cache.region(s, h), ref["region"], t_lens[s], ref["layout"], v_bits, d)


# ---------------------------------------------------------------- decode

def _decode_vs_oracle(wl, t_lens, qz, bank, rv, dtype=torch.float32, append_then_attend=False, pairing=0,
                      theta=None, check_logits=True, check_seqs=None, step_twin=False, levels="fp32",
                      bank_seed=0):
    """Decode over a cache prefilled with the workload's keys and values, against the oracle.
    With append_then_attend the last token of every sequence is appended (bgtq_quantize_append)
    and the query sits at its position.  With step_twin a second cache gets the same prefill and
    the last token through bgtq_decode_step instead; its outputs, logits, cache arrays, lengths
    and status must equal the first cache's bit for bit.  `levels` picks the oracle's
    reconstruction levels ("fp32": the Lloyd-Max centroids the method defines; "fp16": those
    rounded to fp16), one or a tuple.  Returns the cache and the worst relative error seen."""
    dev = _cuda()
    d, h_kv, g = wl.d, wl.h_kv, wl.group
    assert np.array_equal(bank, synth.rotation_bank(d, seed=bank_seed)), "the oracle regenerates the rotations"
    theta = wl.theta if theta is None else theta
    batch = len(t_lens)
    cap = -(-(max(t_lens) + 1) // 64) * 64
    caches = [bgtq.PackedCache(batch, h_kv, d, wl.budget, wl.v_bits, cap, pairing=pairing, device=dev)
              for _ in range(2 if step_twin else 1)]
    tails = []
    for s, t_len in enumerate(t_lens):
        n_pre = t_len - 1 if append_then_attend else t_len
        k = np.stack([synth.keys(wl, s, 0, h, 0, t_len) for h in range(h_kv)])
        v = np.stack([synth.values(wl, s, 0, h, 0, t_len) for h in range(h_kv)])
        if n_pre > 0:
            kt, vt = _t(k[:, :n_pre], dtype), _t(v[:, :n_pre], dtype)
            for c in caches:
                bgtq.bgtq_prefill(qz, c, kt, vt, s)
            del kt, vt
        tails.append((_t(k[:, -1:], dtype), _t(v[:, -1:], dtype)))
        del k, v
    q = _t(np.stack([synth.queries(wl, s, 0) for s in range(batch)]))
    if append_then_attend:
        for s, (kn, vn) in enumerate(tails):
            bgtq.bgtq_quantize_append(qz, caches[0], kn[None], vn[None], seq_begin=s)
    pos = None if append_then_attend else torch.tensor(t_lens, dtype=torch.int64, device=dev)
    out, logits = bgtq.bgtq_decode_attention(qz, caches[0], q, theta, q_pos=pos, logits=True)
    if step_twin:
        assert append_then_attend
        kn = torch.stack([t[0] for t in tails]).contiguous()
        vn = torch.stack([t[1] for t in tails]).contiguous()
        out_b, lg_b = bgtq.bgtq_decode_step(qz, caches[1], q, kn, vn, theta, logits=True)
        torch.cuda.synchronize()
        a, b = caches
        assert torch.equal(a.lengths, b.lengths), "lengths differ"
        assert torch.equal(a.status, b.status), f"status {int(a.status[0])} vs {int(b.status[0])}"
        for name in ("k_codes", "k_norms", "v_codes", "v_norms", "widths", "layouts"):
            assert torch.equal(getattr(a, name), getattr(b, name)), f"decode step cache {name} differs"
        bad = [(s, h) for s in range(batch) for h in range(wl.h_q) if not torch.equal(out[s, h], out_b[s, h])]
        assert not bad, f"decode step output differs from append + decode at (seq, head) {bad[:12]} of {len(bad)}"
        for s, t_len in enumerate(t_lens):
            assert torch.equal(logits[s, :, :t_len], lg_b[s, :, :t_len]), f"decode step logits differ (seq {s})"
        _say(f"  decode step == append + decode, bit for bit ({batch} seqs)")
        del out_b, lg_b
    torch.cuda.synchronize()
    out, logits = out.cpu().numpy(), logits.cpu().numpy()
    cache = caches[0]
    del caches
    qn = q.cpu().numpy()
    jobs, keys = [], []
    for s, t_len in enumerate(t_lens):
        if check_seqs is not None and s not in check_seqs:
            continue
        for h in range(h_kv):
            jobs.append(dict(wl=wl, s=s, h=h, t_len=t_len, n_pre=t_len - 1 if append_then_attend else t_len,
                             dtype="bf16" if dtype == torch.bfloat16 else "f32", bank_seed=bank_seed,
                             qpos=t_len - 1 if append_then_attend else t_len, theta=theta, pairing=pairing,
                             levels=levels, cap=cap))
            keys.append((s, h))
    assert np.array_equal(qn, np.stack([synth.queries(wl, s, 0) for s in range(batch)]))
    lvls = (levels,) if isinstance(levels, str) else tuple(levels)
    for j in jobs:
        j["levels"] = lvls
    worst = {lv: [0.0, 0.0] for lv in lvls}          # output, logit
    for (s, h), res in zip(keys, oracle_heads(jobs)):
        t_len = t_lens[s]
        for lv in lvls:
            o_ref, l_ref = res[lv]
            e_out = rel_err(out[s, h * g:(h + 1) * g], o_ref)
            if check_logits:
                e_log = rel_err(logits[s, h * g:(h + 1) * g, :t_len], l_ref)
                assert np.all(e_log <= TOL), f"{lv} levels, seq {s} head {h}: logit error {e_log} (output {e_out})"
                worst[lv][1] = max(worst[lv][1], float(e_log.max()))
            assert np.all(e_out <= TOL), f"{lv} levels, seq {s} head {h}: output error {e_out}"
            worst[lv][0] = max(worst[lv][0], float(e_out.max()))
    for lv in lvls:
        _say(f"  worst rel err vs the {lv}-level oracle: output {worst[lv][0]:.2e}, logits "
             f"{worst[lv][1]:.2e} ({len(jobs)} heads)")
    return cache, max(max(w) for w in worst.values())


def test_decode_tiny(rot64):
    _say("decode tiny")
    bank, rv, qz = rot64
    _decode_vs_oracle(synth.TINY, [256], qz, bank, rv)


@pytest.mark.parametrize("t_lens", [[1], [63], [64], [65], [1000, 3, 129, 4096]])
def test_decode_ragged_lengths(t_lens, rot128):
    _say(f"decode ragged {t_lens}")
    bank, rv, qz = rot128
    wl = synth.Workload("ragged", 91, d=128, h_q=14, h_kv=2, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=3, v_bits=2, key_dtype="f32", profile="decay", outlier_blocks=2)
    _decode_vs_oracle(wl, t_lens, qz, bank, rv)


@pytest.mark.parametrize("t_lens", [
    [1000, 3, 129, 4096, 64, 65, 2000, 777],      # distinct lengths, not in order
    [700, 3, 700, 4096, 64, 700, 2000, 64],       # equal lengths: ranked in index order
    [(37 * i) % 301 + 2 for i in range(66)],      # more sequences than the pass ranks: index order
], ids=["distinct", "ties", "66seqs"])
def test_decode_batch_whole_remainder_tiles(rot128, t_lens):
    """A batch of at least 16 (sequence, KV head) units, so the streamed pass launches several
    rounds of workgroups, maps grid slots to sequences longest first and hands remaining tiles out
    whole: ragged lengths with partial tiles and lengths below and above one round of waves,
    decode step twin bit for bit, every head against the oracle."""
    _say(f"decode batch of {len(t_lens)} x 2 KV heads, whole remainder tiles")
    bank, rv, qz = rot128
    wl = synth.Workload("wholetiles", 96, d=128, h_q=16, h_kv=2, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay_jitter", outlier_blocks=2)
    _decode_vs_oracle(wl, t_lens, qz, bank, rv, append_then_attend=True, step_twin=True)


@pytest.mark.parametrize("d,k_bits,v_bits,t_lens", [
    (64, 2, 1, [300, 65]),      # the streamed pass, value pairs of width 1
    (128, 2, 4, [300, 65]),     # width 4: pairs from a 32-bit window
    (128, 1, 5, [300, 65]),     # width 5: pairs from a 64-bit window
    (64, 2, 6, [300, 65]),      # width 6: one lookup per code
    (64, 0, 8, [300]),          # width 8 with no key bits (a zero budget)
    (128, 3, 8, [300, 65]),     # too wide for the streamed pass's staging: the tiled pass
])
def test_decode_value_widths(d, k_bits, v_bits, t_lens, rot64, rot128):
    """Decode at every value width class against the oracle: each way the decode passes turn
    value codes into levels (pairs from one or two dwords, single codes)."""
    _say(f"decode d={d} K{k_bits}V{v_bits} {t_lens}")
    bank, rv, qz = rot64 if d == 64 else rot128
    wl = synth.Workload("vwidths", 95, d=d, h_q=8, h_kv=2, theta=1e4, layers=1, seq_lens=tuple(t_lens),
                        k_bits=k_bits, v_bits=v_bits, key_dtype="f32", profile="decay", outlier_blocks=2)
    # with no key bits every logit is 0, and a normwise logit error is 0 / 0: outputs only
    _decode_vs_oracle(wl, t_lens, qz, bank, rv, append_then_attend=True, step_twin=True, check_logits=k_bits > 0)


def test_decode_interleaved_pairing_and_no_rope(rot64):
    _say("decode interleaved / no rope")
    bank, rv, qz = rot64
    wl = synth.Workload("inter", 92, d=64, h_q=2, h_kv=1, theta=1e4, layers=1, seq_lens=(300,),
                        k_bits=2, v_bits=3, key_dtype="f32", profile="decay", outlier_blocks=2)
    _decode_vs_oracle(wl, [300], qz, bank, rv, pairing=1)
    _decode_vs_oracle(wl, [300], qz, bank, rv, theta=0.0)


def test_decode_append_then_attend(rot128):
    _say("decode append-then-attend")
    bank, rv, qz = rot128
    wl = synth.Workload("ata", 93, d=128, h_q=16, h_kv=2, theta=1e6, layers=1, seq_lens=(777,),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay_jitter", outlier_blocks=2)
    _decode_vs_oracle(wl, [777], qz, bank, rv, append_then_attend=True)


def test_decode_llama8b_layer_32k_bf16(rot128):
    """Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, 32K bf16 keys with heavy-tailed outliers, K2V2."""
    _say("decode llama8b 32K bf16")
    bank, rv, qz = rot128
    wl = synth.LLAMA8B_LAYER
    _decode_vs_oracle(wl, list(wl.seq_lens), qz, bank, rv, dtype=torch.bfloat16)


def test_decode_empty_sequence_and_zero_budget(rot64):
    dev = _cuda()
    _say("decode empty sequence / zero K budget")
    bank, rv, qz = rot64
    cache = bgtq.PackedCache(2, 1, 64, 0, 3, 128, device=dev)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1, 50, 64)).astype(np.float32)
    v = rng.standard_normal((1, 50, 64)).astype(np.float32)
    bgtq.bgtq_prefill(qz, cache, _t(k), _t(v), 0)        # sequence 1 stays empty
    q = _t(rng.standard_normal((2, 1, 64)))
    out = bgtq.bgtq_decode_attention(qz, cache, q, 1e4, q_pos=torch.tensor([50, 0], device=dev))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert not out[1].any()
    ref = head_reference(k[0], v[0], 0, 3, bank, rv, 128)
    assert not ref["k_hat"].any()                         # every block dropped: logits all zero
    np.testing.assert_allclose(out[0, 0], ref["v_hat"].mean(0), rtol=0, atol=TOL * np.abs(ref["v_hat"].mean(0)).max())


def test_decode_is_deterministic(rot128):
    _say("decode determinism")
    bank, rv, qz = rot128
    wl = synth.Workload("det", 94, d=128, h_q=8, h_kv=1, theta=1e6, layers=1, seq_lens=(5000,),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay", outlier_blocks=2)
    cache, _ = _decode_vs_oracle(wl, [5000], qz, bank, rv, check_logits=False)
    q = _t(synth.queries(wl, 0, 0)[None])
    a = bgtq.bgtq_decode_attention(qz, cache, q, wl.theta)
    b = bgtq.bgtq_decode_attention(qz, cache, q, wl.theta)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_qwen3b_layer_128k_full_size(rot128):
    """One layer of the Qwen2.5-3B-shaped 128K decode at full size (16 q / 2 kv heads, K3V3), in the
    launch configuration the benchmark times: prefill 131072 tokens, then one decode step
    (bgtq_decode_step: the append as one workgroup beside 127 split workgroups per KV head, the
    wave whose work unit holds the new token waiting for it) on one cache and bgtq_quantize_append +
    bgtq_decode_attention on its twin, bit for bit equal; logits and outputs against the oracle,
    every head."""
    _say("decode qwen3b 128K full size, step and append + decode")
    bank, rv, qz = rot128
    wl = synth.QWEN3B_128K
    _decode_vs_oracle(wl, [wl.seq_lens[0] + 1], qz, bank, rv, append_then_attend=True, check_logits=True,
                      step_twin=True)


def test_decode_qwen3b_layer_512k_full_size(rot128):
    """The same shape at 512K context: prefill 524288 tokens, one decode step (and its append +
    decode twin), attend over 524289; logits and outputs of every head against the oracle."""
    _say("decode qwen3b 512K full size, step and append + decode")
    bank, rv, qz = rot128
    wl = synth.QWEN3B_512K
    _decode_vs_oracle(wl, [wl.seq_lens[0] + 1], qz, bank, rv, append_then_attend=True, check_logits=True,
                      step_twin=True)


def test_decode_qwen7b_ragged_batch_full_size(rot128):
    """One layer of the 7B-Qwen-shaped ragged batch: 16 sequences of 8K..64K tokens, 28 q / 4 kv heads
    (group 7), K3V2, one decode step for all of them (and its append + decode twin); logits and
    outputs of every sequence and head against the oracle."""
    _say("decode qwen7b ragged batch of 16, step and append + decode")
    bank, rv, qz = rot128
    wl = synth.QWEN7B_RAGGED
    _decode_vs_oracle(wl, [t + 1 for t in wl.seq_lens], qz, bank, rv, append_then_attend=True,
                      check_logits=True, step_twin=True)


@pytest.fixture
def valu_decode():
    """Forces the vector-ALU decode kernel (the no-matrix-core path) for one test."""
    old = bgtq.get_option(bgtq.OPT_DECODE_KERNEL)
    bgtq.set_option(bgtq.OPT_DECODE_KERNEL, 1)
    yield
    bgtq.set_option(bgtq.OPT_DECODE_KERNEL, old)


@pytest.mark.parametrize("h_q,h_kv,t_lens", [(16, 2, [4097, 130]), (32, 2, [6000]), (8, 8, [3000])])
def test_decode_valu_kernel_vs_oracle(h_q, h_kv, t_lens, rot128, valu_decode):
    """The vector-ALU decode against the oracle: group 8 (forced; the matrix cores serve it by
    default), group 16 (the only path for it) and group 1, multi-tile ragged lengths."""
    _say(f"decode vector ALU {h_q}/{h_kv} {t_lens}")
    bank, rv, qz = rot128
    wl = synth.Workload("valu", 95, d=128, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay_jitter", outlier_blocks=2)
    _decode_vs_oracle(wl, t_lens, qz, bank, rv, append_then_attend=True, step_twin=True)


@pytest.fixture
def tiled_decode():
    """Forces the tiled matrix-core decode pass (the one that serves caches with a recent-key
    window and geometries the streamed pass does not) for one test."""
    old = bgtq.get_option(bgtq.OPT_DECODE_KERNEL)
    bgtq.set_option(bgtq.OPT_DECODE_KERNEL, 2)
    yield
    bgtq.set_option(bgtq.OPT_DECODE_KERNEL, old)


@pytest.mark.parametrize("h_q,h_kv,t_lens", [(16, 2, [4097, 130]), (8, 8, [3000]), (4, 1, [2, 63, 64, 65])])
def test_decode_tiled_kernel_vs_oracle(h_q, h_kv, t_lens, rot128, tiled_decode):
    """The tiled matrix-core pass against the oracle, with the decode step beside it."""
    _say(f"decode tiled pass {h_q}/{h_kv} {t_lens}")
    bank, rv, qz = rot128
    wl = synth.Workload("tiled", 96, d=128, h_q=h_q, h_kv=h_kv, theta=1e6, layers=1, seq_lens=tuple(t_lens),
                        k_bits=3, v_bits=3, key_dtype="f32", profile="decay_jitter", outlier_blocks=2)
    _decode_vs_oracle(wl, t_lens, qz, bank, rv, append_then_attend=True, step_twin=True)


def test_decode_tiled_kernel_qwen3b_128k(rot128, tiled_decode):
    """The tiled matrix-core pass on the 128K Qwen2.5-3B-shaped layer, every head."""
    _say("decode tiled pass qwen3b 128K")
    bank, rv, qz = rot128
    wl = synth.QWEN3B_128K
    _decode_vs_oracle(wl, [wl.seq_lens[0] + 1], qz, bank, rv, append_then_attend=True, check_logits=True)


def test_decode_valu_kernel_qwen3b_128k(rot128, valu_decode):
    """The vector-ALU decode on the 128K Qwen2.5-3B-shaped layer (group 8), every head."""
    _say("decode vector ALU qwen3b 128K")
    bank, rv, qz = rot128
    wl = synth.QWEN3B_128K
    _decode_vs_oracle(wl, [wl.seq_lens[0] + 1], qz, bank, rv, append_then_attend=True, check_logits=True)
