#!/usr/bin/env python3
"""Benchmark of the hybrid sliding/full GQA attention core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one prefill call of a full-attention layer: batch 1, 8192 tokens,
16 query / 4 KV heads, head_dim 256, RoPE theta 5e6 on the first 64 channels,
causal mask, per-head sigmoid gate (RoPE of Q/K, cache write, attention and
gate: every stage of the prefill path). ``value`` is its algorithmic
throughput in TFLOP/s: 4 * 256 * 16 * (visible query-key pairs) per call
divided by the event-timed duration of the K timed calls.

Decode is timed in its own section after the prefill steps and reported under
"decode": sliding-layer decode over 64 sequences with 512-slot ring caches,
and full-layer decode over 2^20 cached tokens (batch 1) and 8 x 131072
tokens, each as KV GB/s of the attention kernels. Before every timed decode
call a 1 GiB buffer is read so the 256 MB last-level cache cannot serve the
KV cache.

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


def counter_traffic(name, kernel):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when it is missing or the kernel source changed since."""
    p = os.path.join(PROFILES, name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256") != source_sha(KERNEL_SRC[kernel]):
        return None
    return d.get("hbm_bytes_per_launch")


def time_calls(torch, fn, steps, warmup, before=None):
    for _ in range(warmup):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        if before:
            before()
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cpu_baseline(S=8192, n_rows=512):
    """The fp64 oracle on a sample of the headline workload, on host cores."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from full_gqa_attention_spark2_amd import synth
    from oracle import hattn_oracle as O

    inp = synth.prefill_inputs(1, S, 16, 4, seed=0)
    rows = np.linspace(0, S - 1, n_rows).astype(np.int64)
    t0 = time.perf_counter()
    O.prefill_ref(inp["q"], inp["k"], inp["v"], inp["gate"], [0], window=None, theta=5e6, rotary_fraction=0.25,
                  rows=rows)
    dt = time.perf_counter() - t0
    flops = 4 * 256 * 16 * int(sum(int(r) + 1 for r in rows))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n_rows} evenly spaced query rows (all 16 heads, {flops / 1e9:.1f} GFLOP) of the "
                  f"S={S} full-layer prefill, fp64 numpy, {dt:.1f} s on {len(os.sched_getaffinity(0))} "
                  f"visible host cores",
    }


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
    hb.hattn_profile_read(hb.PROFILE_PREFILL)
    hb.hattn_profile_enable(True)
    t_wall = time.perf_counter()
    ms = time_calls(torch, prefill, args.steps, args.warmup)
    t_wall = time.perf_counter() - t_wall
    hb.hattn_profile_enable(False)
    n, attn_total = hb.hattn_profile_read(hb.PROFILE_PREFILL)
    attn_ms = attn_total / max(n, 1)
    log(f"prefill: {ms:.4f} ms/call, attention kernel {attn_ms:.4f} ms over {n} launches, "
        f"{flops / ms / 1e9:.1f} TFLOP/s per call")
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": counter_traffic("prefill_attn_full_s8192_counters.json", "prefill"),
        "kernel": "prefill_attn_kernel", "flop_per_launch": flops, "avg_launch_ms": round(attn_ms, 5),
    }
    del inp, cache, out, ws
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- decode
    decode = None
    if not args.skip_decode:
        decode = {}
        # Reading 1 GiB between calls evicts the KV cache from the 256 MB
        # last-level cache without leaving dirty lines behind.
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)

        def flush_llc():
            torch.sum(flush, dim=0, out=sink)

        def decode_case(tag, desc, B, cap, kind, pos, ck, cv):
            dinp = {k: v.to(dev) for k, v in synth.decode_inputs(B, Hq, Hkv, seed=1).items()}
            pos_d = torch.as_tensor(pos, dtype=torch.int32).to(dev)
            c = hb.KVCache(ck, cv, kind)
            o = torch.empty_like(dinp["q"])
            wsd = torch.empty(max(hb.decode_workspace_size(desc, c, B), 256), dtype=torch.uint8, device=dev)
            maxp = int(max(pos))

            def call():
                hb.hattn_decode(desc, dinp["q"], dinp["k"], dinp["v"], dinp["gate"], pos_d, maxp, c, out=o,
                                workspace=wsd)

            hb.hattn_profile_read(hb.PROFILE_DECODE)
            hb.hattn_profile_enable(True)
            ms_call = time_calls(torch, call, args.steps, args.warmup, before=flush_llc)
            hb.hattn_profile_enable(False)
            n, tot = hb.hattn_profile_read(hb.PROFILE_DECODE)
            k_ms = tot / max(n, 1)
            win = min(cap, 512) if kind == "ring" else None
            toks = sum(min(p + 1, win) if win else p + 1 for p in pos)
            kv_bytes = toks * Hkv * 256 * 2 * 2
            gbps = kv_bytes / (k_ms * 1e-3) / 1e9
            log(f"decode {tag}: kernel {k_ms * 1e3:.1f} us ({n} launches), {gbps:.0f} GB/s, "
                f"{gbps / PEAK_HBM_GBPS * 100:.1f}% of HBM peak")
            decode[tag] = {"GB_per_s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                           "kv_bytes_per_call": kv_bytes, "avg_kernel_us": round(k_ms * 1e3, 2)}

        # sliding layer: batch 64, positions uniform in [512, 2^20), 512-slot rings
        pos = synth.positions_uniform(64, 512, 1 << 20, seed=0).tolist()
        ck = synth.cache_tensor(64, Hkv, 512, seed=100, threads=16).to(dev)
        cv = synth.cache_tensor(64, Hkv, 512, seed=101, threads=16).to(dev)
        decode_case("sliding_b64_ring512", hb.layer_desc("sliding", Hq, Hkv), 64, 512, "ring", pos, ck, cv)
        del ck, cv
        # full layer: batch 1 at position 2^20 - 1, and batch 8 at 131071 (same 4 GiB of KV)
        n = 1 << 20
        ck = synth.cache_tensor(1, Hkv, n, seed=200, threads=16).to(dev)
        cv = synth.cache_tensor(1, Hkv, n, seed=201, threads=16).to(dev)
        full = hb.layer_desc("full", Hq, Hkv)
        decode_case("full_b1_1M", full, 1, n, "linear", [n - 1], ck, cv)
        m = n // 8
        decode_case("full_b8_131072", full, 8, m, "linear", [m - 1] * 8, ck.view(8, Hkv, m, 256),
                    cv.view(8, Hkv, m, 256))
        del ck, cv, flush
        torch.cuda.empty_cache()

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
        "decode": decode,
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
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not "
              "part of this benchmark.", file=sys.stderr)
        return 2
    if "RANK" in os.environ and os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        return 2
    line = run(args)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
