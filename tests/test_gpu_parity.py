"""Parity of the HIP path (through the C ABI) with the CPU fp64 oracle.

Bars: floating-point outputs within max-abs 1e-2 and relative RMS 3e-3 of
the oracle (the headline workloads exactly; other cases widen each element's
max-abs bar by what the bf16 store alone adds above |out| = 2, see
store_allowance); slots, positions and masks bit-exact; cached keys equal to
the oracle's bf16-rounded rotated keys (a last-bit difference is allowed only
on values that sit on a rounding boundary to within the two sides' fp64
cos/sin ulps, which the test bounds).
"""
import os
import sys

import numpy as np
import pytest
import torch

from full_gqa_attention_spark2_amd import binding as hb
from full_gqa_attention_spark2_amd import synth
from oracle import hattn_oracle as O

import parity_log

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
REL_RMS = 3e-3
DEV = "cuda"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def errors(gpu, ref):
    g = O.f64(gpu.float().cpu())
    d = g - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))


def store_allowance(ref):
    """What the bf16 store alone may add to an element's error beyond its
    size at |ref| < 2: half a bf16 ulp of |ref| minus 2^-8 (the half ulp on
    [1, 2)), 0 below 2. Outputs this large only occur in rows that see a
    handful of keys (the first prefill rows, tiny windows)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.maximum(0.0, 2.0 ** (e - 8) - 2.0 ** -8)


def check(tag, gpu, ref, max_abs=MAX_ABS, rel_rms=REL_RMS, strict=False):
    """Max-abs and relative-RMS bars. strict: the plain max-abs bar (the
    headline workloads); otherwise each element's bar is widened by what
    the bf16 store alone adds at its magnitude (store_allowance)."""
    assert torch.isfinite(gpu.float()).all(), f"{tag}: non-finite output"
    ea, er = errors(gpu, ref)
    d = np.abs(O.f64(gpu.float().cpu()) - ref)
    eq = float((d - store_allowance(ref)).max())
    line = (f"[parity] {tag}: max_abs={ea:.3e} (beyond the store's extra rounding {eq:.3e}) "
            f"rel_rms={er:.3e} max|ref|={np.abs(ref).max():.3f}")
    log(line)
    if strict:
        parity_log.record(line)
    assert (ea if strict else eq) <= max_abs and er <= rel_rms, (tag, ea, eq, er)


def check_silu(tag, gpu, ref, gate):
    """The silu gate multiplies the sigmoid-gated output by g (silu(g) =
    g * sigmoid(g)), so outputs reach |g| times the sigmoid case's size and
    their bf16 rounding alone exceeds 1e-2 there. The max-abs bar is scaled
    per (token, head) by max(1, |g|), on top of the store allowance that
    `check` gives outside the headline workloads; the relative RMS bar is
    unchanged."""
    assert torch.isfinite(gpu.float()).all(), f"{tag}: non-finite output"
    d = O.f64(gpu.float().cpu()) - ref
    scale = np.maximum(1.0, np.abs(O.f64(gate)))[..., None]
    ea = float((np.maximum(np.abs(d) - store_allowance(ref), 0.0) / scale).max())
    er = float(np.linalg.norm(d) / np.linalg.norm(ref))
    log(f"[parity] {tag}: max_abs/max(1,|g|)={ea:.3e} rel_rms={er:.3e} max|ref|={np.abs(ref).max():.3f}")
    assert ea <= MAX_ABS and er <= REL_RMS, (tag, ea, er)


def check_bf16_values(tag, gpu_bf16, ref64, max_frac=1e-5):
    """Cached rotated keys: bf16 bits vs the oracle's bf16-rounded values."""
    g = O.f64(gpu_bf16.float().cpu())
    bad = g != ref64
    n = int(bad.sum())
    log(f"[parity] {tag}: {n} of {bad.size} cached values differ")
    if n:
        ulp = np.abs(ref64[bad]) * 2.0 ** -7
        assert np.all(np.abs(g[bad] - ref64[bad]) <= ulp * 1.0001), tag
    assert n <= max(1, max_frac * bad.size), tag


def check_page_params(desc, layer, overrides):
    """The library's defaults for a layer type are the oracle's own page
    parameters (page "Spark-X2.5 架构（4B / 1.7B）" §2 and §4 tables), checked
    before the descriptor drives the oracle."""
    want = O.layer_params(layer)
    if "window" not in overrides:
        assert (desc.window if desc.window > 0 else None) == want["window"], (layer, desc.window)
    if "rope_theta" not in overrides:
        assert desc.rope_theta == want["theta"], (layer, desc.rope_theta)
    if "rotary_fraction" not in overrides:
        assert desc.rotary_fraction == want["rotary_fraction"], (layer, desc.rotary_fraction)
    assert desc.head_dim == O.HEAD_DIM


def to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


# ------------------------------------------------------------------ indices
@pytest.mark.parametrize("kind,layer,cap,p0", [
    ("ring", "sliding", 512, 0), ("ring", "sliding", 512, 5), ("ring", "sliding", 512, 509),
    ("ring", "sliding", 512, 1000), ("ring", "sliding", 512, (1 << 20) - 5),
    ("linear", "full", 700, 0), ("linear", "full", 700, 600),
    ("linear", "sliding", 700, 100), ("linear", "sliding", 1300, 1290),
])
def test_index_probe_bit_exact(kind, layer, cap, p0):
    desc = hb.layer_desc(layer)
    n_q = 4 if kind == "ring" or p0 + 4 <= cap else cap - p0
    mask, kpos, slot = hb.hattn_debug_index_probe(desc, kind, cap, p0, n_q)
    torch.cuda.synchronize()
    w = O.layer_params(layer)["window"]
    for i in range(n_q):
        p = p0 + i
        if kind == "ring":
            want_pos = O.ring_slot_positions(p + 1, cap)
            want_slot = int(O.ring_slot(p, cap))
        else:
            want_pos = O.linear_slot_positions(p + 1, cap)
            want_slot = p
        assert np.array_equal(kpos[i].cpu().numpy(), want_pos)
        assert np.array_equal(mask[i].cpu().numpy().astype(bool), O.allowed(p, want_pos, w))
        assert int(slot[i]) == want_slot


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("layer", ["sliding", "full"])
def test_rope_apply_matches_oracle(layer):
    prm = O.layer_params(layer)
    g = torch.Generator().manual_seed(11)
    x = torch.randn((53, 6, 256), generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 1 << 20, (53,), generator=g, dtype=torch.int32)
    pos[0] = 0
    ref = O.bf16_rne(O.rope(x, pos.numpy(), prm["theta"], prm["rotary_fraction"]))
    xd = x.to(DEV)
    hb.hattn_rope_apply(xd, pos.to(DEV), prm["theta"], prm["rotary_fraction"])
    torch.cuda.synchronize()
    check_bf16_values(f"rope_apply {layer}", xd, ref)
    assert torch.equal(xd[0].cpu(), x[0])  # position 0 is the identity
    r = int(256 * prm["rotary_fraction"])
    assert torch.equal(xd[:, :, r:].cpu(), x[:, :, r:])  # channels past r pass through


def test_gpu_gate_and_window_invariants():
    # the gate: out(g = 0) is exactly half of out(g = +30) (sigmoid(30) is
    # 1.0 in fp32, and halving commutes with the bf16 store)
    desc = hb.layer_desc("full")
    inp = synth.prefill_inputs(1, 200, 16, 4, seed=140)
    outs = []
    for gv in (0.0, 30.0):
        d = to_dev(inp)
        d["gate"] = torch.full_like(d["gate"], gv)
        cache = hb.KVCache.empty(1, 4, 256, "linear")
        outs.append(hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], [0], cache))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], (outs[1].float() * 0.5).to(torch.bfloat16))
    # a window covering every query-key distance cuts nothing: bitwise the
    # result of a far wider window (sliding layers all run the split-query
    # kernel), and the oracle's causal attention at the standard bars
    S = 300
    inp_h = synth.prefill_inputs(1, S, 16, 4, seed=141)
    inp = to_dev(inp_h)
    full = hb.layer_desc("full")
    outs = []
    for w in (S + 7, 1 << 20):
        wide = hb.layer_desc("sliding", rope_theta=full.rope_theta, rotary_fraction=full.rotary_fraction, window=w)
        c = hb.KVCache.empty(1, 4, S, "linear")
        outs.append(hb.hattn_prefill(wide, inp["q"], inp["k"], inp["v"], inp["gate"], [0], c))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    z = torch.zeros(1, 4, S, 256, dtype=torch.bfloat16)
    ref, _ = oracle_prefill(full, inp_h, z, z, [0], "linear", S)
    check("prefill window covering every distance vs causal", outs[0].cpu(), ref)


def test_decode_split_count_does_not_change_the_result():
    # the same four sequences decoded alone (a split plan: several
    # workgroups per sequence, merged) and inside a batch of 64 (one
    # workgroup per sequence): equal up to the order of the sums
    desc = hb.layer_desc("sliding")
    pos = synth.positions_uniform(64, 512, 1 << 20, seed=142).numpy()
    inp = synth.decode_inputs(64, 16, 4, seed=143)
    ck = synth.cache_tensor(64, 4, 512, seed=144)
    cv = synth.cache_tensor(64, 4, 512, seed=145)
    big = hb.KVCache(ck.to(DEV), cv.to(DEV), "ring")
    d = to_dev(inp)
    o64 = hb.hattn_decode(desc, d["q"], d["k"], d["v"], d["gate"], torch.as_tensor(pos).to(DEV), int(pos.max()), big)
    small = hb.KVCache(ck[:4].to(DEV), cv[:4].to(DEV), "ring")
    s4 = {k: v[:4].contiguous() for k, v in d.items()}
    o4 = hb.hattn_decode(desc, s4["q"], s4["k"], s4["v"], s4["gate"], torch.as_tensor(pos[:4]).to(DEV),
                         int(pos[:4].max()), small)
    torch.cuda.synchronize()
    diff = (o4.float() - o64[:4].float()).abs()
    rel = (diff.norm() / o64[:4].float().norm()).item()
    log(f"[parity] split vs wide decode: max diff {diff.max().item():.3e}, relative RMS {rel:.3e}")
    # a tenth of the parity bars: only the order of fp32 sums differs
    assert diff.max().item() <= MAX_ABS / 10 and rel <= REL_RMS / 10
    assert torch.equal(small.k, big.k[:4]) and torch.equal(small.v, big.v[:4])


# ------------------------------------------------------------------ prefill
def run_prefill(layer, B, S, Hq, Hkv, start, seed, cache_kind, cap, hist_seed=None, q_scale=1.0,
                window=None, gate_act="sigmoid"):
    overrides = {"gate_act": gate_act}
    if window is not None:
        overrides["window"] = window
    desc = hb.layer_desc(layer, Hq, Hkv, **overrides)
    check_page_params(desc, layer, overrides)
    inp = synth.prefill_inputs(B, S, Hq, Hkv, seed=seed, q_scale=q_scale)
    if hist_seed is not None:
        ck = synth.cache_tensor(B, Hkv, cap, seed=hist_seed)
        cv = synth.cache_tensor(B, Hkv, cap, seed=hist_seed + 1)
    else:
        ck = torch.zeros((B, Hkv, cap, 256), dtype=torch.bfloat16)
        cv = torch.zeros_like(ck)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), cache_kind)
    d = to_dev(inp)
    out = hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], start, cache)
    torch.cuda.synchronize()
    return desc, inp, ck, cv, cache, out


def history_for(kind, ck, cv, start, cap):
    """The oracle's view of a cache holding positions 0..start[b]-1."""
    B = ck.shape[0]
    n = cap
    hk, hv, hp = [], [], []
    for b in range(B):
        if kind == "ring":
            pos = O.ring_slot_positions(start[b], cap)
        else:
            pos = O.linear_slot_positions(start[b], cap)
        hp.append(pos)
    return ck, cv, np.stack(hp)


def oracle_prefill(desc, inp, ck, cv, start, kind, cap, rows=None):
    w = desc.window if desc.window > 0 else None
    hk, hv, hp = history_for(kind, ck, cv, start, cap)
    return O.prefill_ref(inp["q"], inp["k"], inp["v"], inp["gate"], start, window=w, theta=desc.rope_theta,
                         rotary_fraction=desc.rotary_fraction, hist_k=hk, hist_v=hv, hist_pos=hp, rows=rows,
                         gate_act=O.GATE_ACTS[desc.gate_act])


def cache_after_prefill(ck, cv, k_hat, v, start, kind, cap):
    """The oracle's view of a cache after a prefill: the history ck/cv with
    the new tokens' oracle keys k_hat [B,S,Hkv,D] and values v at their slots
    (position p in slot p, or p mod cap for a ring's last cap tokens)."""
    hk, hv = O.f64(ck).copy(), O.f64(cv).copy()
    B, S = k_hat.shape[:2]
    vv = O.f64(v)
    for b in range(B):
        keep = min(S, cap) if kind == "ring" else S
        for i in range(S - keep, S):
            p = start[b] + i
            slot = p % cap if kind == "ring" else p
            hk[b, :, slot] = k_hat[b, i]
            hv[b, :, slot] = vv[b, i]
    return hk, hv


def test_prefill_sliding_seq1024():
    # one sliding layer: B=1, S=1024, 16/4 heads, theta 1e4 over 256 channels, window 512, seed 0
    desc, inp, ck, cv, cache, out = run_prefill("sliding", 1, 1024, 16, 4, [0], 0, "ring", 512)
    ref, k_hat = oracle_prefill(desc, inp, ck, cv, [0], "ring", 512)
    check("prefill sliding S=1024", out.cpu(), ref, strict=True)
    # the ring keeps positions 512..1023 at slots p mod 512
    slots = np.arange(512, 1024) % 512
    check_bf16_values("ring keys after prefill", cache.k[0, :, slots].cpu().permute(1, 0, 2),
                      k_hat[0, 512:1024])
    assert torch.equal(cache.v[0, :, slots].cpu().permute(1, 0, 2), inp["v"][0, 512:1024])
    # determinism: the same call again gives the same bits
    cache2 = hb.KVCache(torch.zeros_like(cache.k), torch.zeros_like(cache.v), "ring")
    d = to_dev(inp)
    out2 = hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], [0], cache2)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)


def test_prefill_full_seq8192_every_row():
    # one full layer: B=1, S=8192, 16/4 heads, theta 5e6 on the first 64
    # channels, causal: all 8192 rows x 16 heads against the oracle (in row
    # chunks, to bound the oracle's score matrices)
    S = 8192
    desc, inp, ck, cv, cache, out = run_prefill("full", 1, S, 16, 4, [0], 0, "linear", S)
    ref = np.empty((1, S, 16, 256))
    k_hat = None
    for r0 in range(0, S, 2048):
        rows = np.arange(r0, r0 + 2048)
        ref[:, rows], kh = oracle_prefill(desc, inp, ck, cv, [0], "linear", S, rows=rows)
        k_hat = kh if k_hat is None else k_hat
    check("prefill full S=8192 (every row)", out.cpu(), ref, strict=True)
    check_bf16_values("linear keys after prefill", cache.k[0].cpu().permute(1, 0, 2), k_hat[0])
    assert torch.equal(cache.v[0].cpu().permute(1, 0, 2), inp["v"][0])


@pytest.mark.parametrize("layer,B,S,start,cap,kind", [
    ("full", 2, 77, [0, 13], 100, "linear"),          # ragged S, history on b=1
    ("full", 1, 1, [0], 8, "linear"),                 # a single token
    ("sliding", 2, 100, [700, 3], 512, "ring"),       # ring history, partly filled ring
    ("sliding", 1, 1500, [0], 512, "ring"),           # S > window: ring keeps the last 512
    ("sliding", 1, 600, [40], 700, "linear"),         # sliding layer over a linear cache
])
def test_prefill_small_shapes(layer, B, S, start, cap, kind):
    Hq, Hkv = (8, 2) if layer == "full" else (16, 4)
    desc, inp, ck, cv, cache, out = run_prefill(layer, B, S, Hq, Hkv, start, 3, kind, cap, hist_seed=17)
    ref, k_hat = oracle_prefill(desc, inp, ck, cv, start, kind, cap)
    check(f"prefill {layer} B={B} S={S} start={start} {kind}", out.cpu(), ref)
    for b in range(B):
        keep = min(S, cap) if kind == "ring" else S
        pos = np.arange(start[b] + S - keep, start[b] + S)
        slots = pos % cap if kind == "ring" else pos
        check_bf16_values(f"cache keys b={b}", cache.k[b, :, slots].cpu().permute(1, 0, 2),
                          k_hat[b, pos - start[b]])


@pytest.mark.parametrize("fraction", [0.0625, 0.5])
def test_prefill_and_decode_other_rotary_widths(fraction):
    # r = 16 (RoPE partners in the other half of the wave) and 128 (same
    # lane, no specialised prologue): the general query path
    desc = hb.layer_desc("full", rotary_fraction=fraction)
    B, S = 2, 90
    inp = synth.prefill_inputs(B, S, 16, 4, seed=41)
    ck = torch.zeros((B, 4, 128, 256), dtype=torch.bfloat16)
    cv = torch.zeros_like(ck)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), "linear")
    d = to_dev(inp)
    out = hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], [0, 5], cache)
    torch.cuda.synchronize()
    ref, k_hat = oracle_prefill(desc, inp, ck, cv, [0, 5], "linear", 128)
    check(f"prefill rotary fraction {fraction}", out.cpu(), ref)
    # decode of the next token on the same cache
    dinp = synth.decode_inputs(B, 16, 4, seed=42)
    pos = np.array([S, S + 5])
    hk, hv = cache_after_prefill(ck, cv, k_hat, inp["v"], [0, 5], "linear", 128)
    dd = to_dev(dinp)
    o = hb.hattn_decode(desc, dd["q"], dd["k"], dd["v"], dd["gate"], torch.as_tensor(pos, dtype=torch.int32).to(DEV),
                        int(pos.max()), cache)
    torch.cuda.synchronize()
    ref_d, slots, k_hat_d = oracle_decode(desc, dinp, hk, hv, pos, "linear")
    check(f"decode rotary fraction {fraction}", o.cpu(), ref_d)
    check_decode_cache(cache, dinp, slots, k_hat_d)


@pytest.mark.parametrize("layer,kind,cap", [("sliding", "ring", 512), ("full", "linear", 2048)])
def test_varlen_prefill_ragged_batch(layer, kind, cap):
    # eight sequences of 0 .. 600 new tokens over cached histories, in one call
    lens = [0, 1, 77, 300, 31, 64, 129, 600]
    starts = [5, 0, 1000, 3, 511, 700, 2, 40]
    B, T = len(lens), sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    desc = hb.layer_desc(layer)
    inp = {n: t[0] for n, t in synth.prefill_inputs(1, T, 16, 4, seed=90).items()}
    ck = synth.cache_tensor(B, 4, cap, seed=91)
    cv = synth.cache_tensor(B, 4, cap, seed=92)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), kind)
    d = to_dev(inp)
    out = hb.hattn_prefill_varlen(desc, d["q"], d["k"], d["v"], d["gate"], cu, starts, cache)
    torch.cuda.synchronize()
    hk, hv, hp = history_for(kind, ck, cv, starts, cap)
    w = desc.window if desc.window > 0 else None
    ref, k_hat = O.prefill_varlen_ref(inp["q"], inp["k"], inp["v"], inp["gate"], cu, starts, window=w,
                                      theta=desc.rope_theta, rotary_fraction=desc.rotary_fraction,
                                      hist_k=hk, hist_v=hv, hist_pos=hp)
    check(f"varlen prefill {layer} lengths {lens}", out.cpu(), ref)
    for b in range(B):
        n = lens[b]
        if n == 0:
            assert torch.equal(cache.k[b].cpu(), ck[b]) and torch.equal(cache.v[b].cpu(), cv[b])
            continue
        keep = min(n, cap) if kind == "ring" else n
        pos = np.arange(starts[b] + n - keep, starts[b] + n)
        slots = pos % cap if kind == "ring" else pos
        rows = cu[b] + pos - starts[b]
        check_bf16_values(f"varlen cache keys b={b}", cache.k[b, :, slots].cpu().permute(1, 0, 2), k_hat[rows])
        assert torch.equal(cache.v[b, :, slots].cpu().permute(1, 0, 2), inp["v"][rows])


def test_varlen_prefill_with_equal_lengths_is_bitwise_the_batched_call():
    B, S, starts = 3, 100, [0, 50, 700]
    desc = hb.layer_desc("sliding")
    inp = to_dev(synth.prefill_inputs(B, S, 16, 4, seed=93))
    ck = synth.cache_tensor(B, 4, 512, seed=94).to(DEV)
    cv = synth.cache_tensor(B, 4, 512, seed=95).to(DEV)
    c1 = hb.KVCache(ck.clone(), cv.clone(), "ring")
    c2 = hb.KVCache(ck.clone(), cv.clone(), "ring")
    o1 = hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], starts, c1)
    pk = lambda t: t.reshape((B * S,) + tuple(t.shape[2:]))
    o2 = hb.hattn_prefill_varlen(desc, pk(inp["q"]), pk(inp["k"]), pk(inp["v"]), pk(inp["gate"]),
                                 [0, S, 2 * S, 3 * S], starts, c2)
    torch.cuda.synchronize()
    assert torch.equal(pk(o1), o2)
    assert torch.equal(c1.k, c2.k) and torch.equal(c1.v, c2.v)


def test_prefill_window_one_and_peaky():
    desc, inp, ck, cv, cache, out = run_prefill("sliding", 1, 300, 16, 4, [0], 4, "linear", 300, window=1)
    ref, _ = oracle_prefill(desc, inp, ck, cv, [0], "linear", 300)
    check("prefill window=1", out.cpu(), ref)
    # Peaky softmax: queries 8x larger make scores 8x larger, and the score
    # error grows with the query rounding. Sliding layers feed the queries as
    # bf16 high + low parts (~16 significant bits); rows past 511 also see the
    # window cut keys. bf16 queries alone could not meet the
    # bars (the CPU error model's test shows that for any pipeline rounding
    # the queries to bf16). The relative RMS bar is the standard one. The
    # max-abs bar is doubled: where one key dominates a row, its probability
    # is 2^(s - m) against the lazily moved running max m (m moves only by
    # more than 2^8), so it is not exactly 1 and its bf16 rounding (2^-9
    # relative) reaches outputs of size 2-4.
    desc, inp, ck, cv, cache, out = run_prefill("sliding", 1, 768, 16, 4, [0], 5, "ring", 512, q_scale=8.0)
    ref, _ = oracle_prefill(desc, inp, ck, cv, [0], "ring", 512)
    check("prefill peaky softmax (q x8)", out.cpu(), ref, max_abs=2 * MAX_ABS)


def test_chunked_prefill_equals_monolithic():
    S, c = 256, 96
    desc = hb.layer_desc("full")
    inp = to_dev(synth.prefill_inputs(1, S, 16, 4, seed=9))
    whole = hb.KVCache.empty(1, 4, S, "linear")
    o1 = hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], whole)
    parts = hb.KVCache.empty(1, 4, S, "linear")
    sl = lambda t, a, b: t[:, a:b].contiguous()
    oa = hb.hattn_prefill(desc, *(sl(inp[x], 0, c) for x in ("q", "k", "v", "gate")), [0], parts)
    ob = hb.hattn_prefill(desc, *(sl(inp[x], c, S) for x in ("q", "k", "v", "gate")), [c], parts)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], 1), o1)
    assert torch.equal(parts.k, whole.k) and torch.equal(parts.v, whole.v)


# ------------------------------------------------------------------ decode
def run_decode(layer, B, Hq, Hkv, pos, cap, kind, seed, hist_seed, window=None, fill=None,
               gate_act="sigmoid"):
    overrides = {"gate_act": gate_act}
    if window is not None:
        overrides["window"] = window
    desc = hb.layer_desc(layer, Hq, Hkv, **overrides)
    check_page_params(desc, layer, overrides)
    inp = synth.decode_inputs(B, Hq, Hkv, seed=seed)
    ck = synth.cache_tensor(B, Hkv, cap, seed=hist_seed, fill_tokens=fill)
    cv = synth.cache_tensor(B, Hkv, cap, seed=hist_seed + 1, fill_tokens=fill)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), kind)
    d = to_dev(inp)
    pos_t = torch.as_tensor(pos, dtype=torch.int32)
    out = hb.hattn_decode(desc, d["q"], d["k"], d["v"], d["gate"], pos_t.to(DEV), int(pos_t.max()), cache)
    torch.cuda.synchronize()
    return desc, inp, ck, cv, cache, out, pos_t.numpy()


def oracle_decode(desc, inp, ck, cv, pos, kind):
    w = desc.window if desc.window > 0 else None
    return O.decode_ref(inp["q"], inp["k"], inp["v"], inp["gate"], pos, ck, cv, kind=kind, window=w,
                        theta=desc.rope_theta, rotary_fraction=desc.rotary_fraction,
                        gate_act=O.GATE_ACTS[desc.gate_act])


def check_decode_cache(cache, inp, slots, k_hat):
    B = len(slots)
    for b in range(B):
        check_bf16_values(f"decode key b={b}", cache.k[b, :, int(slots[b])].cpu(), k_hat[b])
        assert torch.equal(cache.v[b, :, int(slots[b])].cpu(), inp["v"][b])


def test_decode_sliding_batch64_ring():
    # batch 64, positions uniform in [512, 2^20), 512-slot rings, 16/4 heads
    pos = synth.positions_uniform(64, 512, 1 << 20, seed=0).numpy()
    desc, inp, ck, cv, cache, out, pos = run_decode("sliding", 64, 16, 4, pos, 512, "ring", 0, 100)
    ref, slots, k_hat = oracle_decode(desc, inp, ck, cv, pos, "ring")
    check("decode sliding B=64 ring", out.cpu(), ref, strict=True)
    check_decode_cache(cache, inp, slots, k_hat)


def test_decode_full_1m_tokens():
    # batch 1, query at position 1048575 over a 2^20-token linear cache
    n = 1 << 20
    desc, inp, ck, cv, cache, out, pos = run_decode("full", 1, 16, 4, [n - 1], n, "linear", 1, 200, fill=n - 1)
    ref, slots, k_hat = oracle_decode(desc, inp, ck, cv, pos, "linear")
    check("decode full B=1 L=2^20", out.cpu(), ref, strict=True)
    check_decode_cache(cache, inp, slots, k_hat)


def test_decode_full_batch8_131072():
    n = 131072
    desc, inp, ck, cv, cache, out, pos = run_decode("full", 8, 16, 4, [n - 1] * 8, n, "linear", 2, 300, fill=n - 1)
    ref, slots, k_hat = oracle_decode(desc, inp, ck, cv, pos, "linear")
    check("decode full B=8 L=131072", out.cpu(), ref, strict=True)
    check_decode_cache(cache, inp, slots, k_hat)


def test_decode_partial_ring_and_small_cases():
    # positions below 511: only slots 0..p hold tokens; junk elsewhere
    pos = [0, 3, 300, 510, 511, 512, 1023, 5000]
    desc, inp, ck, cv, cache, out, pos = run_decode("sliding", 8, 16, 4, pos, 512, "ring", 3, 400)
    ref, slots, k_hat = oracle_decode(desc, inp, ck, cv, pos, "ring")
    check("decode partial rings", out.cpu(), ref)
    check_decode_cache(cache, inp, slots, k_hat)
    # 1.7B shape, full layer, ragged positions over a linear cache
    pos = [0, 1, 127, 128, 129, 4095]
    desc, inp, ck, cv, cache, out, pos = run_decode("full", 6, 8, 2, pos, 4096, "linear", 4, 500)
    ref, slots, k_hat = oracle_decode(desc, inp, ck, cv, pos, "linear")
    check("decode full 8/2 ragged", out.cpu(), ref)
    check_decode_cache(cache, inp, slots, k_hat)


def test_silu_gate_mode_prefill_and_decode():
    # the alternative gate activation silu(g) = g * sigmoid(g) (page §3)
    desc, inp, ck, cv, cache, out = run_prefill("sliding", 2, 300, 16, 4, [700, 0], 6, "ring", 512,
                                                hist_seed=60, gate_act="silu")
    ref, _ = oracle_prefill(desc, inp, ck, cv, [700, 0], "ring", 512)
    check_silu("prefill sliding silu gate", out.cpu(), ref, inp["gate"])
    desc, inp, ck, cv, cache, out = run_prefill("full", 1, 200, 16, 4, [1000], 7, "linear", 1200,
                                                hist_seed=62, gate_act="silu")
    ref, _ = oracle_prefill(desc, inp, ck, cv, [1000], "linear", 1200)
    check_silu("prefill full silu gate", out.cpu(), ref, inp["gate"])
    # decode: 256 (sequence, KV head) pairs finish in one workgroup each;
    # one long sequence goes through the cross-workgroup merge
    pos = synth.positions_uniform(64, 512, 1 << 20, seed=8).numpy()
    desc, inp, ck, cv, cache, out, pos = run_decode("sliding", 64, 16, 4, pos, 512, "ring", 9, 64,
                                                    gate_act="silu")
    ref, _, _ = oracle_decode(desc, inp, ck, cv, pos, "ring")
    check_silu("decode ring silu gate", out.cpu(), ref, inp["gate"])
    desc, inp, ck, cv, cache, out, pos = run_decode("full", 1, 16, 4, [20000], 20001, "linear", 10, 66,
                                                    fill=20000, gate_act="silu")
    ref, _, _ = oracle_decode(desc, inp, ck, cv, pos, "linear")
    check_silu("decode linear silu gate (merged splits)", out.cpu(), ref, inp["gate"])


def test_planned_arena_layer_stack():
    # a 4-layer stack (3 sliding, 1 full; page §2 order) planned into one
    # arena by hattn_kv_plan; two prefill chunks and a decode step per layer
    B, T, S1, S2 = 2, 700, 400, 200
    plan, total = hb.hattn_kv_plan(4, 4, B, T)
    arena = hb.kv_arena(total)
    arena.fill_(0xFF)                      # every bf16 reads as NaN until written
    caches = [hb.kv_cache_at(e, arena) for e in plan]
    assert [c.kind for c in caches] == [hb.KV_RING] * 3 + [hb.KV_LINEAR]
    for li in (2, 3):
        desc = hb.layer_desc("full" if li == 3 else "sliding")
        kind = "linear" if li == 3 else "ring"
        cap = plan[li].capacity
        others = [(arena[e.k_offset:e.k_offset + e.bytes // 2].clone(), e) for j, e in enumerate(plan) if j != li]
        inp = synth.prefill_inputs(B, S1 + S2, 16, 4, seed=70 + li)
        d = to_dev(inp)
        sl = lambda t, a, b: t[:, a:b].contiguous()
        o1 = hb.hattn_prefill(desc, *(sl(d[x], 0, S1) for x in ("q", "k", "v", "gate")), [0, 0], caches[li])
        o2 = hb.hattn_prefill(desc, *(sl(d[x], S1, S1 + S2) for x in ("q", "k", "v", "gate")), [S1, S1],
                              caches[li])
        torch.cuda.synchronize()
        # the oracle's monolithic prefill of all S1 + S2 tokens (chunked == monolithic)
        ck = torch.zeros((B, 4, cap, 256), dtype=torch.bfloat16)
        ref, k_hat = oracle_prefill(desc, inp, ck, ck.clone(), [0, 0], kind, cap)
        check(f"arena layer {li} prefill", torch.cat([o1, o2], 1).cpu(), ref)
        # decode of token S1 + S2 on the arena cache
        dinp = synth.decode_inputs(B, 16, 4, seed=80 + li)
        pos = np.array([S1 + S2] * B)
        dd = to_dev(dinp)
        o = hb.hattn_decode(desc, dd["q"], dd["k"], dd["v"], dd["gate"],
                            torch.as_tensor(pos, dtype=torch.int32).to(DEV), S1 + S2, caches[li])
        torch.cuda.synchronize()
        hk, hv = cache_after_prefill(ck, ck.clone(), k_hat, inp["v"], [0, 0], kind, cap)
        ref_d, _, _ = oracle_decode(desc, dinp, hk, hv, pos, kind)
        check(f"arena layer {li} decode", o.cpu(), ref_d)
        # the other layers' K blocks are untouched
        for before, e in others:
            assert torch.equal(arena[e.k_offset:e.k_offset + e.bytes // 2], before)


def _paged_from_linear(lin_k, lin_v, page_size, extra_pages, seed):
    """A paged copy of a linear cache [B, Hkv, cap, D]: the pages go to a
    seeded random permutation of a pool with extra_pages more pages, which
    hold NaN bits (a stray read of them would show)."""
    B, Hkv, cap, D = lin_k.shape
    n = cap // page_size
    num = B * n + extra_pages
    table = np.random.default_rng(seed).permutation(num)[:B * n].reshape(B, n)
    pools = []
    for lin in (lin_k, lin_v):
        pool = torch.full((num, Hkv, page_size, D), float("nan"), dtype=torch.bfloat16)
        for b in range(B):
            for i in range(n):
                pool[table[b, i]] = lin[b, :, i * page_size:(i + 1) * page_size]
        pools.append(pool)
    return pools[0], pools[1], torch.as_tensor(table, dtype=torch.int32)


def _linear_view(cache):
    return (torch.from_numpy(O.paged_to_linear(cache.k.cpu().view(torch.int16).numpy(), cache.block_table.cpu().numpy(),
                                               cache.page_size)).view(torch.bfloat16),
            torch.from_numpy(O.paged_to_linear(cache.v.cpu().view(torch.int16).numpy(), cache.block_table.cpu().numpy(),
                                               cache.page_size)).view(torch.bfloat16))


@pytest.mark.parametrize("B,cap,page,pos", [
    (4, 8192, 256, [8191, 3000, 0, 257]),     # ragged positions, 32 pages per sequence
    (1, 1 << 18, 64, [(1 << 18) - 1]),        # 4096 pages of 64 slots, the per-sequence maximum
])
def test_paged_decode_equals_linear_decode(B, cap, page, pos):
    desc = hb.layer_desc("full")
    inp = to_dev(synth.decode_inputs(B, 16, 4, seed=101))
    ck = synth.cache_tensor(B, 4, cap, seed=102)
    cv = synth.cache_tensor(B, 4, cap, seed=103)
    kp, vp, table = _paged_from_linear(ck, cv, page, 7, seed=104)
    # entries of pages past a sequence's position are never read: fill them with junk
    for b in range(B):
        table[b, pos[b] // page + 1:] = torch.where(torch.arange(table.shape[1] - pos[b] // page - 1) % 2 == 0,
                                                    -7, 1 << 30).to(torch.int32)
    lin = hb.KVCache(ck.to(DEV), cv.to(DEV), "linear")
    pg = hb.KVCache.paged(kp.to(DEV), vp.to(DEV), table.to(DEV))
    pos_t = torch.as_tensor(pos, dtype=torch.int32).to(DEV)
    o_lin = hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos_t, max(pos), lin)
    o_pg = hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos_t, max(pos), pg)
    torch.cuda.synchronize()
    assert torch.equal(o_pg, o_lin)
    dinp = synth.decode_inputs(B, 16, 4, seed=101)
    ref, _, _ = oracle_decode(desc, dinp, ck, cv, np.array(pos), "linear")
    check(f"paged decode B={B} cap={cap} page={page}", o_pg.cpu(), ref)
    # the new rows went to their pages: the paged cache reads back as the linear one
    for b in range(B):
        row = pos[b] % page
        pk = pg.k[int(table[b, pos[b] // page])][:, row].cpu()
        assert torch.equal(pk, lin.k[b, :, pos[b]].cpu())
        assert torch.equal(pg.v[int(table[b, pos[b] // page])][:, row].cpu(), lin.v[b, :, pos[b]].cpu())


def test_paged_chunked_prefill_equals_linear_prefill():
    # a 300-token chunk on top of 1000 / 2900 cached tokens, pages of 128
    B, S, cap, page, starts = 2, 300, 4096, 128, [1000, 2900]
    desc = hb.layer_desc("full")
    inp = synth.prefill_inputs(B, S, 16, 4, seed=105)
    ck = synth.cache_tensor(B, 4, cap, seed=106)
    cv = synth.cache_tensor(B, 4, cap, seed=107)
    kp, vp, table = _paged_from_linear(ck, cv, page, 3, seed=108)
    lin = hb.KVCache(ck.to(DEV), cv.to(DEV), "linear")
    pg = hb.KVCache.paged(kp.to(DEV), vp.to(DEV), table.to(DEV))
    d = to_dev(inp)
    o_lin = hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], starts, lin)
    o_pg = hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], starts, pg)
    torch.cuda.synchronize()
    assert torch.equal(o_pg, o_lin)
    lk, lv = _linear_view(pg)
    assert torch.equal(lk, lin.k.cpu()) and torch.equal(lv, lin.v.cpu())
    ref, _ = oracle_prefill(desc, inp, ck, cv, starts, "linear", cap)
    check("paged chunked prefill", o_pg.cpu(), ref)


def check_block(tag, gpu, ref, x):
    """The block's output is x + y in fp32 (the residual stream, page §5)
    with y = out_proj(...) itself a bf16 module output: an upstream
    difference of any size can move y's rounding by one bf16 ulp. Each
    element's max-abs bar is widened by one ulp of y (y = ref - x, x being
    fp32 values and y bf16 values); the relative RMS bar is unchanged."""
    assert gpu.dtype == torch.float32, f"{tag}: the residual stream is fp32"
    assert torch.isfinite(gpu).all(), f"{tag}: non-finite output"
    g = O.f64(gpu.cpu())
    y = ref - O.f64(x)
    ay = np.abs(y)
    ulp_y = np.where(ay > 0, 2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -126))) - 7), 0.0)
    d = np.abs(g - ref)
    eq = float((d - ulp_y).max())
    er = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
    log(f"[parity] {tag}: max_abs={d.max():.3e} (beyond the rounding of y {eq:.3e}) "
        f"rel_rms={er:.3e} max|ref|={np.abs(ref).max():.3f} max|y|={ay.max():.3f}")
    assert eq <= MAX_ABS and er <= REL_RMS, (tag, d.max(), eq, er)


def _block(hidden, Hq, Hkv, seed):
    w = synth.block_weights(hidden, Hq, Hkv, seed=seed)
    dev = hb.BlockWeights(w["norm"].to(DEV), w["qkvg"].to(DEV), w["o"].to(DEV), rms_eps=1e-6)
    return w, dev


@pytest.mark.parametrize("layer,hidden,Hq,Hkv,kind,cap", [
    ("full", 2560, 16, 4, "linear", 2048),     # the 4B shape
    ("sliding", 2048, 8, 2, "ring", 512),      # the 1.7B shape
    ("sliding", 1024, 4, 1, "ring", 512),      # 1540 fused outputs: rows padded to 1544 for alignment
])
def test_block_prefill_and_decode(layer, hidden, Hq, Hkv, kind, cap):
    # RMSNorm -> fused q/k/v/g projection -> core -> out_proj -> + residual,
    # on a ragged batch over cached histories, then one decode step
    desc = hb.layer_desc(layer, Hq, Hkv)
    w, wd = _block(hidden, Hq, Hkv, seed=120)
    lens, starts = [300, 77, 1], [0, 1000, 5]
    B, T = len(lens), sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = synth.hidden_states(T, hidden, seed=121)
    ck = synth.cache_tensor(B, Hkv, cap, seed=122)
    cv = synth.cache_tensor(B, Hkv, cap, seed=123)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), kind)
    out = hb.hattn_block_prefill(desc, wd, x.to(DEV), cu, starts, cache)
    torch.cuda.synchronize()
    hk, hv, hp = history_for(kind, ck, cv, starts, cap)
    win = desc.window if desc.window > 0 else None
    kw = dict(Hq=Hq, Hkv=Hkv, window=win, theta=desc.rope_theta, rotary_fraction=desc.rotary_fraction)
    ref, k_hat = O.block_prefill_ref(x, w["norm"], w["qkvg"], w["o"], 1e-6, cu, starts, hist_k=hk, hist_v=hv,
                                     hist_pos=hp, **kw)
    check_block(f"block prefill {layer} hidden={hidden}", out.cpu(), ref, x)
    # in place (out is x) gives the same bits
    cache2 = hb.KVCache(ck.to(DEV), cv.to(DEV), kind)
    xi = x.to(DEV)
    hb.hattn_block_prefill(desc, wd, xi, cu, starts, cache2, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi, out)
    # decode of the next token of every sequence on the updated cache
    hk2, hv2 = cache_after_varlen_prefill(ck, cv, k_hat, _v_of_block(x, w, Hq, Hkv), cu, starts, kind, cap)
    xd = synth.hidden_states(B, hidden, seed=124)
    pos = np.array([s + n for s, n in zip(starts, lens)])
    od = hb.hattn_block_decode(desc, wd, xd.to(DEV), torch.as_tensor(pos, dtype=torch.int32).to(DEV),
                               int(pos.max()), cache)
    torch.cuda.synchronize()
    kd = dict(kw)
    kd.pop("window")
    ref_d, _, _ = O.block_decode_ref(xd, w["norm"], w["qkvg"], w["o"], 1e-6, pos, hk2, hv2, kind=kind, window=win,
                                     **kd)
    check_block(f"block decode {layer} hidden={hidden}", od.cpu(), ref_d, xd)


@pytest.mark.parametrize("B", [1, 17, 64, 65])
def test_block_decode_token_counts(B):
    # decode batches of 1, 17 and 64 sequences: the weight-streaming GEMM's
    # partial and full token blocks (its out_proj epilogue adds the
    # residual); 65 sequences: past its limit, hipBLASLt and the separate
    # residual add
    desc = hb.layer_desc("sliding")
    w, wd = _block(2560, 16, 4, seed=150)
    ck = synth.cache_tensor(B, 4, 512, seed=151)
    cv = synth.cache_tensor(B, 4, 512, seed=152)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), "ring")
    pos = synth.positions_uniform(B, 0, 1 << 20, seed=153).numpy()
    x = synth.hidden_states(B, 2560, seed=154)
    out = hb.hattn_block_decode(desc, wd, x.to(DEV), torch.as_tensor(pos).to(DEV), int(pos.max()), cache)
    torch.cuda.synchronize()
    ref, _, _ = O.block_decode_ref(x, w["norm"], w["qkvg"], w["o"], 1e-6, pos, ck, cv, Hq=16, Hkv=4, kind="ring",
                                   window=512, theta=desc.rope_theta, rotary_fraction=desc.rotary_fraction)
    check_block(f"block decode B={B}", out.cpu(), ref, x)
    # in place (out is x): the out_proj epilogue reads each residual element
    # before it writes it, so the bits are the same
    cache2 = hb.KVCache(ck.to(DEV), cv.to(DEV), "ring")
    xi = x.to(DEV)
    hb.hattn_block_decode(desc, wd, xi, torch.as_tensor(pos).to(DEV), int(pos.max()), cache2, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi, out)


def cache_after_varlen_prefill(ck, cv, k_hat, v, cu, start, kind, cap):
    """cache_after_prefill for packed new tokens (sequence b: rows cu[b] ..
    cu[b+1]-1 of k_hat and v)."""
    hk, hv = O.f64(ck).copy(), O.f64(cv).copy()
    vv = O.f64(v)
    for b in range(len(cu) - 1):
        S = cu[b + 1] - cu[b]
        keep = min(S, cap) if kind == "ring" else S
        for i in range(S - keep, S):
            p = start[b] + i
            slot = p % cap if kind == "ring" else p
            hk[b, :, slot] = k_hat[cu[b] + i]
            hv[b, :, slot] = vv[cu[b] + i]
    return hk, hv


def _v_of_block(x, w, Hq, Hkv):
    """The values the block's projection gives for inputs x (the oracle's
    own arithmetic), [T, Hkv, 256]."""
    h = O.rms_norm(x, w["norm"], 1e-6)
    return O.split_qkvg(O.linear_bf16(h, w["qkvg"]), Hq, Hkv)[2]


def test_decode_and_prefill_replay_from_a_captured_hip_graph():
    # serving loops capture the call once and replay it with new positions in
    # device memory: every replay must equal the eager call on the same state
    B = 16
    desc = hb.layer_desc("sliding")
    inp = to_dev(synth.decode_inputs(B, 16, 4, seed=130))
    ck = synth.cache_tensor(B, 4, 512, seed=131).to(DEV)
    cv = synth.cache_tensor(B, 4, 512, seed=132).to(DEV)
    g_cache = hb.KVCache(ck.clone(), cv.clone(), "ring")
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.empty_like(inp["q"])
    ws = torch.empty(max(hb.decode_workspace_size(desc, g_cache, B), 256), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the library's one-time work outside the capture
        hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos, 1 << 20, g_cache, out=out,
                        workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos, 1 << 20, g_cache, out=out,
                        workspace=ws)
    e_cache = hb.KVCache(g_cache.k.clone(), g_cache.v.clone(), "ring")
    for step, p0 in enumerate([600, 601, 5000, 123456]):
        newpos = torch.arange(B, dtype=torch.int32) * 7 + p0
        pos.copy_(newpos.to(DEV))
        graph.replay()
        torch.cuda.synchronize()
        e_out = hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], newpos.to(DEV), 1 << 20, e_cache)
        torch.cuda.synchronize()
        assert torch.equal(out, e_out), step
        assert torch.equal(g_cache.k, e_cache.k) and torch.equal(g_cache.v, e_cache.v), step
    # a prefill call captured and replayed twice over the same inputs
    pdesc = hb.layer_desc("full")
    pin = to_dev(synth.prefill_inputs(1, 300, 16, 4, seed=133))
    pc = hb.KVCache.empty(1, 4, 512, "linear")
    pout = torch.empty_like(pin["q"])
    pws = torch.empty(max(hb.prefill_workspace_size(pdesc, pc, 1, 300), 256), dtype=torch.uint8, device=DEV)
    hb.hattn_prefill(pdesc, pin["q"], pin["k"], pin["v"], pin["gate"], [0], pc, out=pout, workspace=pws)
    torch.cuda.synchronize()
    eager = pout.clone()
    pgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(pgraph):
        hb.hattn_prefill(pdesc, pin["q"], pin["k"], pin["v"], pin["gate"], [0], pc, out=pout, workspace=pws)
    for _ in range(2):
        pout.zero_()
        pgraph.replay()
        torch.cuda.synchronize()
        assert torch.equal(pout, eager)


def test_ring_decode_equals_windowed_linear_decode():
    B, p = 4, 3000
    desc = hb.layer_desc("sliding")
    inp = to_dev(synth.decode_inputs(B, 16, 4, seed=7))
    lin_k = synth.cache_tensor(B, 4, 4096, seed=600)
    lin_v = synth.cache_tensor(B, 4, 4096, seed=601)
    ring_k = torch.zeros((B, 4, 512, 256), dtype=torch.bfloat16)
    ring_v = torch.zeros_like(ring_k)
    src = np.arange(p - 511, p)
    ring_k[:, :, src % 512] = lin_k[:, :, src]
    ring_v[:, :, src % 512] = lin_v[:, :, src]
    pos = torch.full((B,), p, dtype=torch.int32, device=DEV)
    lin = hb.KVCache(lin_k.to(DEV), lin_v.to(DEV), "linear")
    ring = hb.KVCache(ring_k.to(DEV), ring_v.to(DEV), "ring")
    o_lin = hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos, p, lin)
    o_ring = hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos, p, ring)
    torch.cuda.synchronize()
    d = (o_lin.float() - o_ring.float()).abs().max().item()
    log(f"[parity] ring vs windowed-linear decode max diff {d:.3e}")
    assert d <= 2 * 2.0 ** -8 * o_lin.float().abs().max().item()
    assert torch.equal(ring.k[:, :, p % 512], lin.k[:, :, p])


def test_decode_equals_prefill_row():
    S = 300
    desc = hb.layer_desc("full")
    inp = to_dev(synth.prefill_inputs(1, S, 16, 4, seed=12))
    c1 = hb.KVCache.empty(1, 4, S, "linear")
    full = hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], c1)
    c2 = hb.KVCache.empty(1, 4, S, "linear")
    sl = lambda t: t[:, :S - 1].contiguous()
    hb.hattn_prefill(desc, sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["gate"]), [0], c2)
    pos = torch.tensor([S - 1], dtype=torch.int32, device=DEV)
    last = lambda t: t[:, S - 1].contiguous()
    dec = hb.hattn_decode(desc, last(inp["q"]), last(inp["k"]), last(inp["v"]), last(inp["gate"]), pos, S - 1, c2)
    torch.cuda.synchronize()
    d = (dec.float() - full[:, S - 1].float()).abs().max().item()
    log(f"[parity] decode vs prefill row max diff {d:.3e}")
    assert d <= 1e-2
    assert torch.equal(c1.k, c2.k) and torch.equal(c1.v, c2.v)


def test_decode_out_of_range_position_gives_nan_and_no_write():
    desc = hb.layer_desc("full")
    inp = to_dev(synth.decode_inputs(2, 16, 4, seed=8))
    cache = hb.KVCache.empty(2, 4, 64, "linear")
    pos = torch.tensor([5, 40], dtype=torch.int32, device=DEV)
    out = hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos, 10, cache)
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all() and torch.isfinite(out[0].float()).all()
    assert not cache.k[1].any() and cache.k[0, :, 5].any()


def test_decode_wide_grid_partial_rings_and_invalid_positions():
    # 64 sequences x 4 KV heads reach the one-workgroup-per-pair decode grid;
    # mix partial rings, full rings and positions outside [0, max_pos]
    B = 64
    rng = np.random.default_rng(11)
    pos = rng.integers(0, 5000, B).astype(np.int64)
    pos[:8] = [0, 1, 17, 255, 510, 511, 512, 4999]
    pos[20], pos[41] = -1, 6000  # invalid: negative, and above max_pos below
    max_pos = 5000
    desc = hb.layer_desc("sliding")
    inp = synth.decode_inputs(B, 16, 4, seed=12)
    ck = synth.cache_tensor(B, 4, 512, seed=800)
    cv = synth.cache_tensor(B, 4, 512, seed=801)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), "ring")
    d = to_dev(inp)
    out = hb.hattn_decode(desc, d["q"], d["k"], d["v"], d["gate"], torch.as_tensor(pos, dtype=torch.int32).to(DEV),
                          max_pos, cache)
    torch.cuda.synchronize()
    bad = np.array([20, 41])
    good = np.setdiff1d(np.arange(B), bad)
    assert torch.isnan(out[bad].float()).all()
    assert torch.equal(cache.k[bad].cpu(), ck[bad]) and torch.equal(cache.v[bad].cpu(), cv[bad])
    sub = {k: v[good] for k, v in inp.items()}
    ref, slots, k_hat = O.decode_ref(sub["q"], sub["k"], sub["v"], sub["gate"], pos[good], ck[good], cv[good],
                                     kind="ring", window=512, theta=desc.rope_theta,
                                     rotary_fraction=desc.rotary_fraction)
    check("decode wide grid (64 x 4 pairs), partial rings", out[good].cpu(), ref)
    for i, b in enumerate(good[:8]):
        check_bf16_values(f"decode key b={b}", cache.k[b, :, int(slots[i])].cpu(), k_hat[i])


def _poisoned(c, valid):
    """A copy of cache tensor c whose slots outside `valid` ([B, cap] bool)
    hold NaN in K-like and +Inf in V-like tensors: memory a caller never
    wrote may hold any bits, and no such slot may reach the output."""
    g = c.clone()
    bits = g.view(torch.int16)
    bad = torch.as_tensor(~valid)[:, None, :, None].expand_as(bits)
    bits[bad] = 0x7FC0
    bits[1::2][bad[1::2]] = 0x7F80   # odd sequences get +Inf instead
    return g


def test_unwritten_cache_slots_holding_nan_or_inf_are_never_read():
    # decode over partial rings and over a linear cache, slot p itself
    # poisoned too (the kernel writes the new token there before use)
    for layer, kind, cap, pos in [("sliding", "ring", 512, [0, 5, 300, 510]),
                                  ("full", "linear", 1000, [0, 63, 64, 700])]:
        B = len(pos)
        desc = hb.layer_desc(layer)
        inp = synth.decode_inputs(B, 16, 4, seed=31)
        ck = synth.cache_tensor(B, 4, cap, seed=900)
        cv = synth.cache_tensor(B, 4, cap, seed=901)
        valid = np.arange(cap)[None, :] < np.asarray(pos)[:, None]
        cache = hb.KVCache(_poisoned(ck, valid).to(DEV), _poisoned(cv, valid).to(DEV), kind)
        d = to_dev(inp)
        out = hb.hattn_decode(desc, d["q"], d["k"], d["v"], d["gate"], torch.as_tensor(pos, dtype=torch.int32).to(DEV),
                              max(pos), cache)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all(), f"decode {kind}: non-finite output"
        ref, slots, k_hat = oracle_decode(desc, inp, ck, cv, np.asarray(pos), kind)
        check(f"decode {kind} over poisoned unwritten slots", out.cpu(), ref)
        check_decode_cache(cache, inp, slots, k_hat)
    # prefill: a linear cache and a ring whose slots past the history are poisoned
    for layer, kind, cap, start, S in [("full", "linear", 200, [0, 100], 50), ("sliding", "ring", 512, [0, 300], 40)]:
        B = len(start)
        desc = hb.layer_desc(layer)
        inp = synth.prefill_inputs(B, S, 16, 4, seed=32)
        ck = synth.cache_tensor(B, 4, cap, seed=902)
        cv = synth.cache_tensor(B, 4, cap, seed=903)
        valid = np.arange(cap)[None, :] < np.asarray(start)[:, None]
        clean_k = torch.where(torch.as_tensor(valid)[:, None, :, None], ck, torch.zeros_like(ck))
        clean_v = torch.where(torch.as_tensor(valid)[:, None, :, None], cv, torch.zeros_like(cv))
        cache = hb.KVCache(_poisoned(ck, valid).to(DEV), _poisoned(cv, valid).to(DEV), kind)
        d = to_dev(inp)
        out = hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], start, cache)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all(), f"prefill {kind}: non-finite output"
        ref, _ = oracle_prefill(desc, inp, clean_k, clean_v, start, kind, cap)
        check(f"prefill {kind} over poisoned unwritten slots", out.cpu(), ref)


def test_profiling_hook_counts_and_times_kernel_sections():
    # the event pairs the bench reads: one per call while enabled, none after
    desc = hb.layer_desc("full")
    inp = to_dev(synth.prefill_inputs(1, 64, 16, 4, seed=51))
    cache = hb.KVCache.empty(1, 4, 64, "linear")
    hb.hattn_profile_read(hb.PROFILE_PREFILL)
    hb.hattn_profile_read(hb.PROFILE_DECODE)
    hb.hattn_profile_enable(True)
    try:
        for _ in range(3):
            hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], cache)
        dinp = to_dev(synth.decode_inputs(1, 16, 4, seed=52))
        big = hb.KVCache.empty(1, 4, 128, "linear")
        hb.hattn_decode(desc, dinp["q"], dinp["k"], dinp["v"], dinp["gate"],
                        torch.tensor([100], dtype=torch.int32, device=DEV), 100, big)
    finally:
        hb.hattn_profile_enable(False)
    n, ms = hb.hattn_profile_read(hb.PROFILE_PREFILL)
    assert n == 3 and ms > 0.0
    n, ms = hb.hattn_profile_read(hb.PROFILE_DECODE)
    assert n == 1 and ms > 0.0
    hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], cache)
    torch.cuda.synchronize()
    assert hb.hattn_profile_read(hb.PROFILE_PREFILL) == (0, 0.0)


def test_lds_probe_reports_plausible_rates():
    # the bench's LDS ceiling: every block records its shader clock ticks;
    # reads per clock and cycles per MFMA within what a CU can do
    out = torch.zeros(256, 2, dtype=torch.int64, device=DEV)
    for mode, iters, per_round in ((0, 200, 32768), (1, 200, 16384), (2, 50, None)):
        out.zero_()
        hb.debug_lds_probe(mode, 256, iters, out)
        torch.cuda.synchronize()
        ticks = out[:, 0].double()
        assert bool((ticks > 0).all()), mode
        med = float(ticks.median())
        if per_round:
            bpc = iters * per_round / med
            print(f"LDS probe mode {mode}: {bpc:.1f} B per clock per CU", flush=True)
            assert 16.0 < bpc <= 1024.0
        else:
            cpm = med / (iters * 64)
            print(f"LDS probe mode 2: {cpm:.2f} cycles per MFMA", flush=True)
            assert 16.0 <= cpm < 400.0


def test_profiling_hook_reads_the_prefill_shader_clock():
    # the clock the bench reports for its timed launches: a plausible MI355X
    # shader clock while profiling, reset by each read, nothing recorded with
    # profiling off; the stamps change no output bit
    desc = hb.layer_desc("full")
    inp = to_dev(synth.prefill_inputs(1, 512, 16, 4, seed=53))
    cache = hb.KVCache.empty(1, 4, 512, "linear")
    plain = hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], cache)
    hb.hattn_profile_enable(True)
    try:
        stamped = hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], cache)
        ghz = hb.hattn_profile_read_clock()
    finally:
        hb.hattn_profile_enable(False)
    hb.hattn_profile_read(hb.PROFILE_PREFILL)
    print(f"prefill shader clock while profiled: {ghz:.3f} GHz", flush=True)
    assert 0.3 < ghz < 3.5
    assert torch.equal(plain, stamped)
    assert hb.hattn_profile_read_clock() == 0.0
    hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0], cache)
    assert hb.hattn_profile_read_clock() == 0.0


# ------------------------------------------------------------------ chunked prefill, 1.7B shape
@pytest.mark.parametrize("layer", ["full", "sliding"])
def test_chunked_prefill_1p7b_shape_sampled(layer):
    # 8/2 heads, batch 2, a 4096-token chunk appended to a 262144-token context
    B, S, s0 = 2, 4096, 262144
    if layer == "full":
        cap, kind, fill = s0 + S, "linear", s0
    else:
        cap, kind, fill = 512, "ring", None
    desc = hb.layer_desc(layer, 8, 2)
    inp = synth.prefill_inputs(B, S, 8, 2, seed=21)
    ck = synth.cache_tensor(B, 2, cap, seed=700, fill_tokens=fill)
    cv = synth.cache_tensor(B, 2, cap, seed=701, fill_tokens=fill)
    cache = hb.KVCache(ck.to(DEV), cv.to(DEV), kind)
    d = to_dev(inp)
    out = hb.hattn_prefill(desc, d["q"], d["k"], d["v"], d["gate"], [s0, s0], cache)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(64), rng.integers(0, S, 64)]))
    ref, k_hat = oracle_prefill(desc, inp, ck, cv, [s0, s0], kind, cap, rows=rows)
    check(f"chunked prefill 1.7B {layer} (sampled rows)", out[:, rows].cpu(), ref, strict=True)


# ------------------------------------------------------------------ seeded sweep
def _sweep_case(rng):
    """One random small configuration within the documented limits."""
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = 4 * Hkv
    layer = str(rng.choice(["sliding", "full"]))
    frac = float(rng.choice([0.0625, 0.125, 0.25, 0.5, 1.0]))
    theta = float(rng.choice([1e4, 5e6, 123.0]))
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 160, B)]
    if sum(lens) == 0:
        lens[0] = 1
    if layer == "sliding":
        w = int(rng.choice([1, 2, 31, 64, 65, 200, 512]))
        kind = str(rng.choice(["ring", "linear"]))
    else:
        w = None
        kind = str(rng.choice(["linear", "paged"]))
    gate_act = str(rng.choice(["sigmoid", "silu"]))
    starts = [int(x) for x in rng.integers(0, 900, B)]
    cap = w if kind == "ring" else max(s + n for s, n in zip(starts, lens)) + 8
    page = None
    if kind == "paged":
        page = int(rng.choice([64, 128]))
        cap = -(-cap // page) * page
    return dict(Hq=Hq, Hkv=Hkv, layer=layer, frac=frac, theta=theta, B=B, lens=lens, w=w, kind=kind,
                starts=starts, cap=cap, page=page, gate_act=gate_act)


@pytest.mark.parametrize("seed", range(32))
def test_seeded_sweep_of_small_configurations(seed):
    # random shapes, windows, rotary widths, thetas, gate modes, ragged
    # lengths and cache kinds (ring, linear, paged); a ragged prefill over a
    # random history, then one decode step
    c = _sweep_case(np.random.default_rng(1000 + seed))
    over = dict(rotary_fraction=c["frac"], rope_theta=c["theta"], gate_act=c["gate_act"])
    if c["w"] is not None:
        over["window"] = c["w"]
    desc = hb.layer_desc(c["layer"], c["Hq"], c["Hkv"], **over)
    B, lens, starts, cap, kind = c["B"], c["lens"], c["starts"], c["cap"], c["kind"]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    inp = {n: t[0] for n, t in synth.prefill_inputs(1, T, c["Hq"], c["Hkv"], seed=2000 + seed).items()}
    ck = synth.cache_tensor(B, c["Hkv"], cap, seed=3000 + seed)
    cv = synth.cache_tensor(B, c["Hkv"], cap, seed=4000 + seed)
    if kind == "paged":
        kp, vp, table = _paged_from_linear(ck, cv, c["page"], 2, seed=6000 + seed)
        cache = hb.KVCache.paged(kp.to(DEV), vp.to(DEV), table.to(DEV))
    else:
        cache = hb.KVCache(ck.to(DEV), cv.to(DEV), kind)
    okind = "linear" if kind == "paged" else kind   # the oracle's view of a paged cache
    d = to_dev(inp)
    out = hb.hattn_prefill_varlen(desc, d["q"], d["k"], d["v"], d["gate"], cu, starts, cache)
    torch.cuda.synchronize()
    hk, hv, hp = history_for(okind, ck, cv, starts, cap)
    ref, k_hat = O.prefill_varlen_ref(inp["q"], inp["k"], inp["v"], inp["gate"], cu, starts, window=c["w"],
                                      theta=c["theta"], rotary_fraction=c["frac"], hist_k=hk, hist_v=hv,
                                      hist_pos=hp, gate_act=c["gate_act"])
    tag = f"sweep {seed}: {c}"
    chk = (lambda t, g, r, gl: check_silu(t, g, r, gl)) if c["gate_act"] == "silu" else \
        (lambda t, g, r, gl: check(t, g, r))
    chk(tag + " prefill", out.cpu(), ref, inp["gate"])
    # the next token of every sequence
    hk2, hv2 = cache_after_varlen_prefill(ck, cv, k_hat, inp["v"], cu, starts, okind, cap)
    pos = np.array([s + n for s, n in zip(starts, lens)])
    dinp = synth.decode_inputs(B, c["Hq"], c["Hkv"], seed=5000 + seed)
    dd = to_dev(dinp)
    o = hb.hattn_decode(desc, dd["q"], dd["k"], dd["v"], dd["gate"], torch.as_tensor(pos, dtype=torch.int32).to(DEV),
                        int(pos.max()), cache)
    torch.cuda.synchronize()
    ref_d, slots, k_hat_d = oracle_decode(desc, dinp, hk2, hv2, pos, okind)
    chk(tag + " decode", o.cpu(), ref_d, dinp["gate"])
    if kind != "paged":
        check_decode_cache(cache, dinp, slots, k_hat_d)
    else:
        lk, lv = _linear_view(cache)
        for b in range(B):
            check_bf16_values(f"{tag} paged key b={b}", lk[b, :, int(slots[b])], k_hat_d[b])
            assert torch.equal(lv[b, :, int(slots[b])], dinp["v"][b])


def test_largest_positions_and_batch():
    # positions at the top of the documented range (just below 2^30), where
    # the RoPE angle reaches ~1e9 rad, and the largest prefill batch (128)
    top = (1 << 30) - 1
    desc = hb.layer_desc("sliding")
    pos = np.array([top, top - 511, (1 << 29) + 7, 512])
    desc_, inp, ck, cv, cache, out, pos = run_decode("sliding", 4, 16, 4, pos, 512, "ring", 160, 161)
    ref, slots, k_hat = oracle_decode(desc_, inp, ck, cv, pos, "ring")
    check("decode at positions near 2^30", out.cpu(), ref)
    check_decode_cache(cache, inp, slots, k_hat)
    # a 300-token prefill ending at 2^30 - 1 over a full ring
    S = 300
    desc_, inp, ck, cv, cache, out = run_prefill("sliding", 1, S, 16, 4, [top + 1 - S], 162, "ring", 512,
                                                 hist_seed=163)
    ref, _ = oracle_prefill(desc_, inp, ck, cv, [top + 1 - S], "ring", 512)
    check("prefill ending at 2^30 - 1", out.cpu(), ref)
    # 128 sequences of 0..9 new tokens in one ragged call (full layer, 8/2 heads)
    rng = np.random.default_rng(164)
    lens = [int(x) for x in rng.integers(0, 10, 128)]
    starts = [int(x) for x in rng.integers(0, 200, 128)]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    fdesc = hb.layer_desc("full", 8, 2)
    pin = {n: t[0] for n, t in synth.prefill_inputs(1, T, 8, 2, seed=165).items()}
    fk = synth.cache_tensor(128, 2, 256, seed=166)
    fv = synth.cache_tensor(128, 2, 256, seed=167)
    fc = hb.KVCache(fk.to(DEV), fv.to(DEV), "linear")
    d = to_dev(pin)
    o = hb.hattn_prefill_varlen(fdesc, d["q"], d["k"], d["v"], d["gate"], cu, starts, fc)
    torch.cuda.synchronize()
    hk, hv, hp = history_for("linear", fk, fv, starts, 256)
    ref, _ = O.prefill_varlen_ref(pin["q"], pin["k"], pin["v"], pin["gate"], cu, starts, window=None,
                                  theta=fdesc.rope_theta, rotary_fraction=fdesc.rotary_fraction, hist_k=hk, hist_v=hv,
                                  hist_pos=hp)
    check("ragged prefill of 128 sequences", o.cpu(), ref)


_SERIAL_SCRIPT = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
from full_gqa_attention_spark2_amd import binding as hb, synth
torch.cuda.set_device(0)
dev = "cuda"
desc = hb.layer_desc("full")
inp = {k: v.to(dev) for k, v in synth.prefill_inputs(2, 200, 16, 4, seed=170).items()}
cache = hb.KVCache.empty(2, 4, 4096, "linear")
out = hb.hattn_prefill(desc, inp["q"], inp["k"], inp["v"], inp["gate"], [0, 3000], cache)
d = {k: v.to(dev) for k, v in synth.decode_inputs(2, 16, 4, seed=171).items()}
pos = torch.tensor([200, 3200], dtype=torch.int32, device=dev)
dout = hb.hattn_decode(desc, d["q"], d["k"], d["v"], d["gate"], pos, 3200, cache)
torch.cuda.synchronize()
np.savez(sys.argv[2], prefill=out.view(torch.int16).cpu().numpy(), decode=dout.view(torch.int16).cpu().numpy(),
         k=cache.k.view(torch.int16).cpu().numpy())
"""


def test_launch_blocking_rerun_is_bitwise_identical(tmp_path):
    # the same prefill and decode (split plan, so two kernels) in a child
    # process with every launch serialised (HIP_LAUNCH_BLOCKING=1) and in a
    # child with the default asynchronous launches: a race between the
    # library's kernels would show as a difference
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "serial.py"
    script.write_text(_SERIAL_SCRIPT)
    res = {}
    for tag, blocking in (("async", None), ("blocking", "1")):
        env = dict(os.environ)
        env.pop("HIP_LAUNCH_BLOCKING", None)
        if blocking:
            env["HIP_LAUNCH_BLOCKING"] = blocking
        f = tmp_path / f"{tag}.npz"
        r = subprocess.run([sys.executable, str(script), root, str(f)], env=env, capture_output=True, text=True,
                           timeout=240)
        assert r.returncode == 0, r.stderr[-2000:]
        res[tag] = np.load(f)
    for name in ("prefill", "decode", "k"):
        assert np.array_equal(res["async"][name], res["blocking"][name]), name
