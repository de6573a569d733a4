#!/usr/bin/env python3
"""Benchmark of the hybrid sliding/full GQA attention core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one prefill call of a full-attention layer: batch 1, 8192 tokens,
16 query / 4 KV heads, head_dim 256, RoPE theta 5e6 on the first 64 channels,
causal mask, per-head sigmoid gate (RoPE of Q/K, cache write, attention and
gate: every stage of the prefill path). ``value`` is its algorithmic
throughput in TFLOP/s: 4 * 256 * 16 * (visible query-key pairs) per call
divided by the event-timed duration of the K timed calls.

Two more prefill workloads are reported under "prefill_configs" (not in
``value``): a sliding layer at 1024 tokens (batch 1, ring cache), and the
1.7B shape's chunked prefill (8 / 2 heads, batch 2, a 4096-token chunk on a
262144-token context), timed as whole 28-layer passes in the page's layer
order over 28 distinct caches (the sum of one call per layer type is kept as
a secondary figure), plus its full layer on a paged cache; and the 4B
attention block (norm, projections, core, out_proj, residual) for prefill and
decode.

Decode is timed in its own section after the prefill steps and reported under
"decode": sliding-layer decode over 64 sequences with 512-slot ring caches,
and full-layer decode over 2^20 cached tokens (batch 1) and 8 x 131072
tokens, each as KV GB/s per call (decode kernel plus split merge, timed
back to back). The calls cycle over enough distinct caches that the 256 MB
last-level cache cannot serve the KV cache.

"roofline" describes the prefill attention kernel (HIP events around each of
its launches in the timed steps), with the shader clock those launches ran at
(stamped by the kernel's workgroups through the library's profiling hook) and
the fraction of peak at that clock, and with the HBM traffic and MFMA-busy
fraction from the committed rocprofv3 counter passes when the kernel source
still matches them. "practical_ceilings" times the library's streaming-read and
MFMA probes and torch's bf16 GEMM beside the path. "cpu_baseline" times the
fp64 oracle on the host on a bounded sample of each workload.

All inputs are seeded synthetic tensors (N(0,1) bf16 Q/K/V and caches, gate
logits N(0, 2^2)) already resident in HBM when timing starts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s + decode KV GB/s (% of MI355X peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
NOMINAL_SCLK_GHZ = 2.4      # the clock that peak assumes (256 CUs x 4096 flop/clk)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = {
    "prefill": os.path.join(ROOT, "full_gqa_attention_spark2_amd", "csrc", "hattn_prefill.hip"),
    "decode": os.path.join(ROOT, "full_gqa_attention_spark2_amd", "csrc", "hattn_decode.hip"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(n_q, start, window=None, n_hist=0):
    """Visible (query, key) pairs of n_q queries at start..start+n_q-1 over a
    cache holding every earlier position (closed form per query)."""
    total = 0
    for i in range(n_q):
        p = start + i
        total += (p + 1) if window is None else min(p + 1, window)
    return total


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_traffic(workload):
    """HBM bytes per launch of a workload's dominant kernel, from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the same
    counters on a copy of known size), or None when the summary is missing or
    the kernel's source has changed since it was taken."""
    p = os.path.join(PROFILES, "hbm_traffic_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get("workloads", {}).get(workload)
    if not e or e.get("source_sha256") != source_sha(KERNEL_SRC[e["source"]]):
        return None
    return e.get("hbm_bytes_per_launch")


def counter_clock():
    """The prefill kernel's average shader clock and MFMA-busy fraction from
    the committed rocprofv3 counter pass (GRBM_GUI_ACTIVE per XCD over the
    dispatch time; SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles), or None
    when the summary is missing or the kernel's source has changed since.
    The profiler serialises those launches, with idle time between them, so
    their clock can differ from that of back-to-back launches
    (shader_clock_GHz in the roofline)."""
    p = os.path.join(PROFILES, "prefill_mfma_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    src = d.get("source")
    if src not in KERNEL_SRC or d.get("source_sha256") != source_sha(KERNEL_SRC[src]):
        return None
    return {"sclk_GHz": d.get("avg_clock_GHz"), "mfma_busy": d.get("mfma_busy"), "dispatches": d.get("dispatches"),
            "source": "profiles/prefill_mfma_counters.json"}


def copy_calibration():
    """A plain device copy of known size (fp32 negation, 1 GiB read + 1 GiB
    written per launch), run under the same counters as the kernels to scale
    FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch

    dev = torch.device("cuda:0")
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"kernel": "torch.neg fp32", "bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
            "launches": 3}


def block_bench(torch, hb, synth, dev, args):
    """The attention block around the core (RMSNorm, fused q/k/v/g
    projection, core, out_proj, residual) on the 4B shape with random
    weights: the full-layer prefill of 8192 tokens and a 64-sequence sliding
    decode."""
    S, Hq, Hkv = 8192, 16, 4
    flops = 4 * 256 * Hq * visible_pairs(S, 0)
    Hd = 2560
    bw = {k: v.to(dev) for k, v in synth.block_weights(Hd, Hq, Hkv, seed=60).items()}
    wts = hb.BlockWeights(bw["norm"], bw["qkvg"], bw["o"], rms_eps=1e-6)
    xb = synth.hidden_states(S, Hd, seed=61).to(dev)
    ob = torch.empty_like(xb)
    cb = hb.KVCache.empty(1, Hkv, S, "linear")
    dfull = hb.layer_desc("full", Hq, Hkv)
    n1 = (Hq + 2 * Hkv) * 256 + Hq
    wsb = torch.empty(hb.block_prefill_workspace_size(dfull, wts, cb, [0, S]), dtype=torch.uint8, device=dev)
    tb = time_each(torch, lambda: hb.hattn_block_prefill(dfull, wts, xb, [0, S], [0], cb, out=ob, workspace=wsb),
                   max(args.steps // 2, 5), 2)
    gemm_fl = 2 * S * Hd * n1 + 2 * S * Hq * 256 * Hd
    blk_fl = gemm_fl + flops
    log(f"block prefill (4B, 8192 tokens): {tb['median']:.3f} ms, "
        f"{blk_fl / (tb['median'] * 1e-3) / 1e12:.1f} TFLOP/s (GEMMs + attention)")
    Bd = 64
    pos = synth.positions_uniform(Bd, 512, 1 << 20, seed=0)
    cr = hb.KVCache(synth.cache_tensor(Bd, Hkv, 512, seed=62, threads=16).to(dev),
                    synth.cache_tensor(Bd, Hkv, 512, seed=63, threads=16).to(dev), "ring")
    xd = synth.hidden_states(Bd, Hd, seed=64).to(dev)
    od = torch.empty_like(xd)
    dsl = hb.layer_desc("sliding", Hq, Hkv)
    pos_d = pos.to(torch.int32).to(dev)
    wsd = torch.empty(hb.block_decode_workspace_size(dsl, wts, cr, Bd), dtype=torch.uint8, device=dev)
    td = time_each(torch, lambda: hb.hattn_block_decode(dsl, wts, xd, pos_d, int(pos.max()), cr, out=od,
                                                        workspace=wsd),
                   max(args.steps, 20), args.warmup)
    log(f"block decode (4B sliding, batch 64): {td['median'] * 1e3:.1f} us per call")
    res = {
        "prefill_s8192_full_ms": {k: round(v, 4) for k, v in tb.items()},
        "prefill_flop": blk_fl, "prefill_gemm_flop": gemm_fl,
        "prefill_TFLOP_per_s": round(blk_fl / (tb["median"] * 1e-3) / 1e12, 2),
        "decode_b64_sliding_us": {k: round(v * 1e3, 2) for k, v in td.items()},
        "weights": "random, N(0, 0.02^2) projections, RMSNorm weight 1 + N(0, 0.1^2)"}
    del bw, wts, xb, ob, cb, wsb, cr, xd, od, wsd
    torch.cuda.empty_cache()
    return res


def to_paged(torch, hb, ck, cv, page, seed):
    """A paged copy of linear caches [B, Hkv, cap, 256]: the B * cap / page
    pages in a seeded random order in one pool, and the block table that
    maps them back."""
    B, H, cap, D = ck.shape
    n = cap // page
    perm = torch.randperm(B * n, generator=torch.Generator().manual_seed(seed))

    def pool(x):
        p = torch.empty((B * n, H, page, D), dtype=x.dtype, device=x.device)
        p[perm.to(x.device)] = x.view(B, H, n, page, D).permute(0, 2, 1, 3, 4).reshape(B * n, H, page, D)
        return p

    return hb.KVCache.paged(pool(ck), pool(cv), perm.view(B, n).to(torch.int32).to(ck.device))


def ceilings(torch, hb, dev, steps=5):
    """What the chip itself delivers, timed beside the path (event-timed,
    back to back): the library's plain streaming-read probe over 4 GiB and
    over 8 distinct 128 MiB buffers in turn (the sliding decode's size and
    grid), back-to-back bf16 MFMA on every CU (with the shader clock over
    it), the LDS read rate of the prefill kernel's fragment reads (alone and
    mixed with its MFMAs, on the shader clock) and torch's bf16 GEMM of
    8192^3 (hipBLASLt)."""
    res = {}
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    big = torch.empty(1 << 30, dtype=torch.int32, device=dev).random_()  # 4 GiB
    sweep = []
    for blocks in (256, 512, 1024, 2048, 4096):
        ms = time_calls(torch, lambda: hb.debug_read_probe(big, blocks, sink), steps, 2)
        sweep.append({"blocks": blocks, "ms": round(ms, 4), "GB_per_s": round(4 * big.numel() / (ms * 1e-3) / 1e9, 1)})
    res["read_4GiB_probe"] = max(sweep, key=lambda r: r["GB_per_s"])
    res["read_4GiB_probe_sweep"] = sweep
    del big
    sets = [torch.empty(1 << 25, dtype=torch.int32, device=dev).random_() for _ in range(8)]  # 8 x 128 MiB
    for blocks in (256, 1024):
        it = [0]

        def rd():
            hb.debug_read_probe(sets[it[0] % 8], blocks, sink)
            it[0] += 1

        ms = time_calls(torch, rd, 8 * steps, 8)
        res[f"read_8x128MiB_probe_{blocks}_blocks"] = {"us": round(ms * 1e3, 2),
                                                      "GB_per_s": round((1 << 27) / (ms * 1e-3) / 1e9, 1)}
    del sets
    fsink = torch.zeros(256 * 4, dtype=torch.float32, device=dev)
    iters = 8000
    hb.debug_mfma_probe(256, iters, fsink)
    ms = time_calls(torch, lambda: hb.debug_mfma_probe(256, iters, fsink), steps, 1)
    fl = 256 * 4 * iters * 8 * 32768
    tf = fl / (ms * 1e-3) / 1e12
    # one 32x32x16 MFMA per 32 cycles per SIMD at full issue: the clock the
    # rate implies (1,024 SIMDs x 1,024 flop per cycle)
    res["mfma_bf16_32x32x16_probe"] = {"ms": round(ms, 4), "TFLOP_per_s": round(tf, 1),
                                       "implied_sclk_GHz": round(tf * 1e12 / (1024 * 1024) / 1e9, 3)}
    # LDS: bytes per shader clock and CU for the prefill kernel's fragment
    # reads, and the prefill step's reads mixed with its MFMAs (cycles per
    # MFMA; 32 when the matrix core never waits), one block per CU
    out = torch.zeros(256, 2, dtype=torch.int64, device=dev)
    lds = {}
    for mode, name, iters_l, per_round in ((0, "ds_read_b128", 4000, 32768), (1, "ds_read_b64_tr_b16", 4000, 16384),
                                           (2, "prefill_step_reads_with_mfma", 500, None)):
        hb.debug_lds_probe(mode, 256, iters_l, out)
        torch.cuda.synchronize()
        ticks = float(out[:, 0].double().median())
        if per_round:
            lds[name] = {"B_per_clock_per_CU": round(iters_l * per_round / ticks, 1), "waves_per_CU": 4}
        else:
            lds[name] = {"cycles_per_mfma": round(ticks / (iters_l * 64), 2), "reads_per_mfma": 1.5, "waves_per_CU": 4}
    res["lds_probe"] = lds
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    ms = time_calls(torch, lambda: torch.mm(a, b), steps, 2)
    res["gemm_bf16_8192_torch_mm"] = {"ms": round(ms, 4), "TFLOP_per_s": round(2 * 8192 ** 3 / (ms * 1e-3) / 1e12, 1)}
    del a, b
    torch.cuda.empty_cache()
    return res


def chunked_stack(torch, hb, synth, dev, passes, warmup):
    """The 1.7B shape's chunked prefill as one 28-layer pass: layers in the
    page's order (sliding, sliding, sliding, full) x 7, each with its own
    cache (21 rings of 512 slots, 7 linear caches of 266,240 slots holding
    262,144 cached tokens), batch 2, 8 / 2 heads, a 4096-token chunk at
    position 262,144. One event pair brackets each whole pass."""
    B, S5, s0, Hq, Hkv = 2, 4096, 262144, 8, 2
    order = ["full" if i % 4 == 3 else "sliding" for i in range(28)]
    desc = {t: hb.layer_desc(t, Hq, Hkv) for t in ("sliding", "full")}
    inp = {t: {k: v.to(dev) for k, v in synth.prefill_inputs(B, S5, Hq, Hkv, seed=40 + 10 * i).items()}
           for i, t in enumerate(("sliding", "full"))}
    out = {t: torch.empty_like(inp[t]["q"]) for t in inp}
    ring_k = synth.cache_tensor(B, Hkv, 512, seed=41, threads=16).to(dev)
    ring_v = synth.cache_tensor(B, Hkv, 512, seed=42, threads=16).to(dev)
    lin_k = synth.cache_tensor(B, Hkv, s0 + S5, seed=51, fill_tokens=s0, threads=16).to(dev)
    lin_v = synth.cache_tensor(B, Hkv, s0 + S5, seed=52, fill_tokens=s0, threads=16).to(dev)
    caches = []
    for t in order:
        if t == "sliding":
            caches.append(hb.KVCache(ring_k.clone(), ring_v.clone(), "ring"))
        else:
            caches.append(hb.KVCache(lin_k.clone(), lin_v.clone(), "linear"))
    del ring_k, ring_v, lin_k, lin_v
    ws = {t: torch.empty(max(hb.prefill_workspace_size(desc[t], caches[order.index(t)], B, S5), 256),
                         dtype=torch.uint8, device=dev) for t in desc}
    starts = [s0] * B

    def one_pass():
        for t, c in zip(order, caches):
            d = inp[t]
            hb.hattn_prefill(desc[t], d["q"], d["k"], d["v"], d["gate"], starts, c, out=out[t], workspace=ws[t])

    t = time_each(torch, one_pass, passes, warmup)
    fl = {tt: 4 * 256 * Hq * B * visible_pairs(S5, s0, window=512 if tt == "sliding" else None) for tt in desc}
    flop = sum(fl[tt] for tt in order)
    del caches, inp, out, ws
    torch.cuda.empty_cache()
    return t, flop, fl


def time_calls(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_each(torch, fn, steps, warmup):
    """Per-call event times (ms): median, p10, p90."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    pick = lambda f: t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9)}


def cpu_baseline(S=8192, budget_s=10.0, n_1m=1 << 20, s0=262144):
    """The fp64 oracle, as it stands, on the host cores.

    Headline (C2, the full-layer prefill of 8192 tokens): interleaved sets
    of 512 evenly spaced query rows (rows k, k+16, k+32, ... for k = 0, 1,
    ...) until about ``budget_s`` seconds of CPU work are done or every row
    is covered. ``per_config`` times the oracle on the other workloads, each
    on a stated bounded sample, in the unit of its GPU figure (TFLOP/s of
    algorithmic attention work, or GB/s of KV read for decode)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from full_gqa_attention_spark2_amd import synth
    from oracle import hattn_oracle as O

    inp = synth.prefill_inputs(1, S, 16, 4, seed=0)
    stride = 16
    done_rows = 0
    flops = 0
    t0 = time.perf_counter()
    for k in range(stride):
        rows = np.arange(k, S, stride, dtype=np.int64)
        O.prefill_ref(inp["q"], inp["k"], inp["v"], inp["gate"], [0], window=None, theta=5e6,
                      rotary_fraction=0.25, rows=rows)
        done_rows += len(rows)
        flops += 4 * 256 * 16 * int((rows + 1).sum())
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    ncores = len(os.sched_getaffinity(0))
    line = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done_rows} of the {S} query rows (interleaved sets of {S // stride} evenly spaced rows, "
                  f"all 16 heads, {flops / 1e9:.1f} GFLOP) of the full-layer prefill, fp64 numpy, "
                  f"{dt:.1f} s on {ncores} visible host cores",
    }
    del inp
    per = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    def exact64(t):
        """The bf16 tensor's values as fp64 numpy (exact), prepared outside
        the timed region so that only the oracle's arithmetic is timed."""
        return t.float().numpy().astype(np.float64)

    # C1: the whole sliding-layer prefill (1024 tokens from position 0)
    c1 = synth.prefill_inputs(1, 1024, 16, 4, seed=30)
    dt = timed(lambda: O.prefill_ref(c1["q"], c1["k"], c1["v"], c1["gate"], [0], window=512, theta=1e4,
                                     rotary_fraction=1.0))
    fl = 4 * 256 * 16 * visible_pairs(1024, 0, window=512)
    per["sliding_s1024"] = {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "seconds": round(dt, 3),
                            "sample": "the whole workload"}
    # C3: the whole sliding decode (64 sequences, full 512-slot rings)
    pos = synth.positions_uniform(64, 512, 1 << 20, seed=0).tolist()
    d3 = synth.decode_inputs(64, 16, 4, seed=1)
    rk = exact64(synth.cache_tensor(64, 4, 512, seed=100, threads=16))
    rv = exact64(synth.cache_tensor(64, 4, 512, seed=101, threads=16))
    dt = timed(lambda: O.decode_ref(d3["q"], d3["k"], d3["v"], d3["gate"], pos, rk, rv, kind="ring", window=512,
                                    theta=1e4, rotary_fraction=1.0))
    kv = 64 * 512 * 4 * 256 * 2 * 2
    per["sliding_b64_ring512"] = {"value": round(kv / dt / 1e9, 3), "unit": "GB/s of KV", "seconds": round(dt, 3),
                                  "sample": "the whole workload"}
    del rk, rv
    # C4a / C4b: one KV head (its 4 query heads) of the full-layer decode
    for tag, n, note in (("full_b1_1M", n_1m, f"1 of the 4 KV heads (its 4 query heads) over {n_1m} positions"),
                         ("full_b8_131072", 1 << 17, "1 of the 8 sequences, 1 of its 4 KV heads, over 131,072 "
                                                     "positions")):
        dq = synth.decode_inputs(1, 4, 1, seed=1)
        ck = exact64(synth.cache_tensor(1, 1, n, seed=200, threads=16))
        cv = exact64(synth.cache_tensor(1, 1, n, seed=201, threads=16))
        dt = timed(lambda: O.decode_ref(dq["q"], dq["k"], dq["v"], dq["gate"], [n - 1], ck, cv, kind="linear",
                                        window=None, theta=5e6, rotary_fraction=0.25))
        kv = n * 256 * 2 * 2
        per[tag] = {"value": round(kv / dt / 1e9, 3), "unit": "GB/s of KV", "seconds": round(dt, 3), "sample": note}
        del ck, cv
    # C5: 32 query rows of sequence 0 per layer type, all 8 heads, over the
    # full history; extrapolated to the 28-layer pass (2 x 4096 rows per
    # layer, 21 sliding + 7 full layers)
    S5, nr = 4096, 32
    rows = np.linspace(0, S5 - 1, nr).astype(np.int64)
    c5 = synth.prefill_inputs(1, S5, 8, 2, seed=50)
    hk = exact64(synth.cache_tensor(1, 2, s0, seed=51, threads=16))
    hv = exact64(synth.cache_tensor(1, 2, s0, seed=52, threads=16))
    hp = np.arange(s0, dtype=np.int64)[None]
    dt_full = timed(lambda: O.prefill_ref(c5["q"], c5["k"], c5["v"], c5["gate"], [s0], window=None, theta=5e6,
                                          rotary_fraction=0.25, hist_k=hk, hist_v=hv, hist_pos=hp, rows=rows))
    del hk, hv
    rk = exact64(synth.cache_tensor(1, 2, 511, seed=41, threads=16))
    rv = exact64(synth.cache_tensor(1, 2, 511, seed=42, threads=16))
    rp = np.arange(s0 - 511, s0, dtype=np.int64)[None]
    dt_sl = timed(lambda: O.prefill_ref(c5["q"], c5["k"], c5["v"], c5["gate"], [s0], window=512, theta=1e4,
                                        rotary_fraction=1.0, hist_k=rk, hist_v=rv, hist_pos=rp, rows=rows))
    scale = 2 * S5 / nr
    est = (7 * dt_full + 21 * dt_sl) * scale
    fl28 = 2 * 4 * 256 * 8 * (7 * visible_pairs(S5, s0) + 21 * visible_pairs(S5, s0, window=512))
    per["chunked_1p7b_28_layers"] = {
        "value": round(fl28 / est / 1e12, 5), "unit": "TFLOP/s", "extrapolated_seconds_28_layers": round(est, 1),
        "sample": f"{nr} query rows of sequence 0 for each layer type, all 8 heads, full history; extrapolated "
                  f"x{scale:.0f} rows x (7 full + 21 sliding layers) (extrapolated)",
        "measured_seconds": {"full_layer_rows": round(dt_full, 3), "sliding_layer_rows": round(dt_sl, 3)}}
    line["per_config"] = per
    return line


def run(args):
    import torch

    from full_gqa_attention_spark2_amd import binding as hb
    from full_gqa_attention_spark2_amd import synth

    hb.lib()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    # ---------------------------------------------------------------- prefill
    S, Hq, Hkv = 8192, 16, 4
    desc = hb.layer_desc("full", Hq, Hkv)
    inp = {k: v.to(dev) for k, v in synth.prefill_inputs(1, S, Hq, Hkv, seed=0).items()}
    cache = hb.KVCache.empty(1, Hkv, S, "linear", device=dev)
    out = torch.empty_like(inp["q"])
    ws = torch.empty(hb.prefill_workspace_size(desc, cache, 1, S), dtype=torch.uint8, device=dev)

    def prefill():
        hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], cache, out=out, workspace=ws)

    flops = 4 * 256 * Hq * visible_pairs(S, 0)
    # warm-up first, then the profiling hook records only the timed calls
    for _ in range(args.warmup):
        prefill()
    torch.cuda.synchronize()
    hb.hattn_profile_read(hb.PROFILE_PREFILL)
    hb.hattn_profile_enable(True)
    ms = time_calls(torch, prefill, args.steps, 0)
    hb.hattn_profile_enable(False)
    n, attn_total = hb.hattn_profile_read(hb.PROFILE_PREFILL)
    sclk = hb.hattn_profile_read_clock()  # the same timed launches
    attn_ms = attn_total / max(n, 1)
    log(f"prefill: {ms:.4f} ms/call, attention kernel {attn_ms:.4f} ms over {n} launches, "
        f"{flops / ms / 1e9:.1f} TFLOP/s per call")
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": counter_traffic("prefill_full_s8192"),
        "kernel": "prefill_attn_kernel", "flop_per_launch": flops, "avg_launch_ms": round(attn_ms, 5),
        "launches_timed": n,
        # shader clock of the timed launches (per workgroup, s_memtime against
        # the fixed-rate s_memrealtime), and the fraction of the bf16 peak at
        # that clock (the published peak assumes 2.4 GHz)
        "shader_clock_GHz": round(sclk, 3),
        "frac_at_shader_clock": round(achieved / (PEAK_BF16_TFLOPS * sclk / NOMINAL_SCLK_GHZ), 4) if sclk > 0 else None,
        "clock_from_counters": counter_clock(),
    }
    del inp, cache, out, ws
    torch.cuda.empty_cache()

    # ------------------------------------------------ other prefill workloads
    prefill_configs = None
    if not args.skip_prefill_configs:
        prefill_configs = {}

        def prefill_case(layer, B, S_, Hq_, Hkv_, s0, cap, kind, fill, seed, steps, warmup, page=None):
            d = hb.layer_desc(layer, Hq_, Hkv_)
            pin = {k: v.to(dev) for k, v in synth.prefill_inputs(B, S_, Hq_, Hkv_, seed=seed).items()}
            c = hb.KVCache(synth.cache_tensor(B, Hkv_, cap, seed=seed + 1, fill_tokens=fill, threads=16).to(dev),
                           synth.cache_tensor(B, Hkv_, cap, seed=seed + 2, fill_tokens=fill, threads=16).to(dev),
                           kind)
            if page:
                c = to_paged(torch, hb, c.k, c.v, page, seed + 3)
            o = torch.empty_like(pin["q"])
            w = torch.empty(max(hb.prefill_workspace_size(d, c, B, S_), 256), dtype=torch.uint8, device=dev)
            starts = [s0] * B

            def call():
                hb.hattn_prefill(d, pin["q"], pin["k"], pin["v"], pin["gate"], starts, c, out=o, workspace=w)

            t = time_each(torch, call, steps, warmup)
            win = 512 if layer == "sliding" else None
            fl = 4 * 256 * Hq_ * B * visible_pairs(S_, s0, window=win)
            return t, fl

        # sliding layer, batch 1, 1024 tokens from position 0 (empty ring)
        t, fl = prefill_case("sliding", 1, 1024, Hq, Hkv, 0, 512, "ring", 0, 30, max(args.steps, 20), args.warmup)
        tf = fl / (t["median"] * 1e-3) / 1e12
        log(f"prefill sliding_s1024: {t['median'] * 1e3:.1f} us per call (median), {tf:.1f} TFLOP/s")
        prefill_configs["sliding_s1024"] = {
            "us_per_call": {k: round(v * 1e3, 2) for k, v in t.items()}, "flop_per_call": fl,
            "TFLOP_per_s": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    if prefill_configs is not None and not args.skip_chunked:
        # 1.7B shape: 8 / 2 heads, batch 2, a 4096-token chunk at 262144:
        # the 28-layer pass measured as a whole, and each layer type alone
        s0, S5 = 262144, 4096
        t28, fl28, _ = chunked_stack(torch, hb, synth, dev, max(5, args.steps // 4), 1)
        ms28 = t28["median"]
        tf28 = fl28 / (ms28 * 1e-3) / 1e12
        log(f"prefill 1.7B chunk, 28-layer pass (measured): {ms28:.2f} ms median "
            f"(p10 {t28['p10']:.2f}, p90 {t28['p90']:.2f}), {tf28:.1f} TFLOP/s")
        ts, fls = prefill_case("sliding", 2, S5, 8, 2, s0, 512, "ring", None, 40, 5, 2)
        torch.cuda.empty_cache()
        tfu, flf = prefill_case("full", 2, S5, 8, 2, s0, s0 + S5, "linear", s0, 50, 5, 2)
        torch.cuda.empty_cache()
        ms28c = 21 * ts["median"] + 7 * tfu["median"]
        log(f"prefill 1.7B chunk, composed 21 x sliding + 7 x full: {ms28c:.2f} ms "
            f"(sliding layer {ts['median']:.3f} ms, full layer {tfu['median']:.3f} ms)")
        # the same full-layer call on a paged cache (pages of 256 slots in a
        # shuffled pool)
        tpg, _ = prefill_case("full", 2, S5, 8, 2, s0, s0 + S5, "linear", s0, 50, 5, 2, page=256)
        torch.cuda.empty_cache()
        log(f"prefill 1.7B full layer, paged cache (256-slot pages): {tpg['median']:.3f} ms "
            f"({flf / (tpg['median'] * 1e-3) / 1e12:.1f} TFLOP/s)")
        prefill_configs["chunked_1p7b_full_layer_paged256"] = {
            "ms": {k: round(v, 4) for k, v in tpg.items()}, "flop": flf,
            "TFLOP_per_s": round(flf / (tpg["median"] * 1e-3) / 1e12, 2),
            "linear_cache_ms": round(tfu["median"], 4)}
        prefill_configs["chunked_1p7b_28_layers"] = {
            "ms_28_layers": round(ms28, 3), "flop_28_layers": fl28, "TFLOP_per_s": round(tf28, 2),
            "frac_bf16_peak": round(tf28 / PEAK_BF16_TFLOPS, 4),
            "measured": "median of whole 28-layer passes (one event pair per pass) over 28 distinct caches",
            "pass_ms": {k: round(v, 3) for k, v in t28.items()},
            "composed_ms_28_layers": round(ms28c, 3),
            "composed_from": "21 x sliding-layer call + 7 x full-layer call, medians (secondary)",
            "sliding_layer_ms": {k: round(v, 4) for k, v in ts.items()}, "sliding_layer_flop": fls,
            "full_layer_ms": {k: round(v, 4) for k, v in tfu.items()}, "full_layer_flop": flf,
            "full_layer_TFLOP_per_s": round(flf / (tfu["median"] * 1e-3) / 1e12, 2)}

    if prefill_configs is not None and not args.skip_block:
        prefill_configs["block_4b"] = block_bench(torch, hb, synth, dev, args)

    # ---------------------------------------------------------------- decode
    # Each decode workload is timed as K back-to-back calls (decode kernel and
    # split merge) between one event pair. Calls cycle over enough distinct KV
    # caches (>= 1 GiB in total) that the 256 MB last-level cache cannot
    # serve a call's KV from the previous ones.
    decode = None
    if not args.skip_decode:
        decode = {}

        def decode_case(tag, desc, B, cap, kind, pos, caches):
            dinp = {k: v.to(dev) for k, v in synth.decode_inputs(B, Hq, Hkv, seed=1).items()}
            pos_d = torch.as_tensor(pos, dtype=torch.int32).to(dev)
            o = torch.empty_like(dinp["q"])
            maxp = int(max(pos))
            cs = [c if isinstance(c, hb.KVCache) else hb.KVCache(c[0], c[1], kind) for c in caches]
            wsd = torch.empty(max(hb.decode_workspace_size(desc, cs[0], B), 256), dtype=torch.uint8, device=dev)
            it = [0]

            def call():
                c = cs[it[0] % len(cs)]
                it[0] += 1
                hb.hattn_decode(desc, dinp["q"], dinp["k"], dinp["v"], dinp["gate"], pos_d, maxp, c, out=o,
                                workspace=wsd)

            steps = max(args.steps, 2 * len(cs))
            ms_call = time_calls(torch, call, steps, args.warmup)
            each = time_each(torch, call, max(steps, 3 * len(cs)), 0)
            win = min(cap, 512) if kind == "ring" else None
            toks = sum(min(p + 1, win) if win else p + 1 for p in pos)
            kv_bytes = toks * Hkv * 256 * 2 * 2
            gbps = kv_bytes / (ms_call * 1e-3) / 1e9
            log(f"decode {tag}: {ms_call * 1e3:.1f} us per call over {steps} calls ({len(cs)} caches), "
                f"{gbps:.0f} GB/s, {gbps / PEAK_HBM_GBPS * 100:.1f}% of HBM peak")
            decode[tag] = {"GB_per_s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                           "kv_bytes_per_call": kv_bytes, "avg_call_us": round(ms_call * 1e3, 2),
                           "per_call_us": {k: round(v * 1e3, 2) for k, v in each.items()},
                           "calls": steps, "distinct_caches": len(cs),
                           "traffic": counter_traffic("decode_" + tag)}

        # sliding layer: batch 64, positions uniform in [512, 2^20), 512-slot
        # rings; eight cache sets of 128 MiB
        pos = synth.positions_uniform(64, 512, 1 << 20, seed=0).tolist()
        sets = [(synth.cache_tensor(64, Hkv, 512, seed=100 + 2 * i, threads=16).to(dev),
                 synth.cache_tensor(64, Hkv, 512, seed=101 + 2 * i, threads=16).to(dev)) for i in range(8)]
        decode_case("sliding_b64_ring512", hb.layer_desc("sliding", Hq, Hkv), 64, 512, "ring", pos, sets)
        del sets
        # full layer: batch 1 at position 2^20 - 1, and batch 8 at 131071
        # (the same 4 GiB of KV, 16x the last-level cache)
        n = 1 << 20
        ck = synth.cache_tensor(1, Hkv, n, seed=200, threads=16).to(dev)
        cv = synth.cache_tensor(1, Hkv, n, seed=201, threads=16).to(dev)
        full = hb.layer_desc("full", Hq, Hkv)
        decode_case("full_b1_1M", full, 1, n, "linear", [n - 1], [(ck, cv)])
        m = n // 8
        decode_case("full_b8_131072", full, 8, m, "linear", [m - 1] * 8,
                    [(ck.view(8, Hkv, m, 256), cv.view(8, Hkv, m, 256))])
        # the 1M-token decode on a paged copy (4096 pages of 256 slots, shuffled)
        pg = to_paged(torch, hb, ck, cv, 256, 7)
        del ck, cv
        torch.cuda.empty_cache()
        decode_case("full_b1_1M_paged256", full, 1, n, "paged", [n - 1], [pg])
        del pg
        torch.cuda.empty_cache()

    ceil = None if args.skip_ceilings else ceilings(torch, hb, dev)
    if ceil:
        log(f"ceilings: {json.dumps(ceil)}")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "full-attention layer prefill: batch 1, seq 8192, 16 Q / 4 KV heads, head_dim 256, "
                        "RoPE theta 5e6 on 64 channels, causal, sigmoid head gate",
            "batch": 1, "seq_len": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": 256,
            "flop_per_step": flops,
        },
        "roofline": roofline,
        "practical_ceilings": ceil,
        "decode": decode,
        "prefill_configs": prefill_configs,
    }
    if not args.skip_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    return line


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-prefill-configs", action="store_true",
                    help="skip the sliding 1024-token and 1.7B chunked prefill timings")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-chunked", action="store_true",
                    help="skip the 1.7B chunked prefill timings (28-layer pass, per layer type, paged)")
    ap.add_argument("--skip-block", action="store_true", help="skip the attention-block timings")
    ap.add_argument("--skip-ceilings", action="store_true",
                    help="skip the read / MFMA probe and GEMM timings")
    ap.add_argument("--ceilings", action="store_true",
                    help="only time the read / MFMA probes and the GEMM (for kernel traces)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the copy of known size used to scale HBM counters")
    ap.add_argument("--block-only", action="store_true",
                    help="only time the attention block around the core (for kernel traces)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not "
              "part of this benchmark.", file=sys.stderr)
        return 2
    if "RANK" in os.environ and os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        line = copy_calibration()
    elif args.ceilings:
        import torch
        from full_gqa_attention_spark2_amd import binding as hb
        line = ceilings(torch, hb, torch.device("cuda:0"), steps=max(args.steps, 5))
    elif args.block_only:
        import torch
        from full_gqa_attention_spark2_amd import binding as hb, synth
        line = block_bench(torch, hb, synth, torch.device("cuda:0"), args)
    else:
        line = run(args)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
