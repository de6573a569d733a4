"""Pins of the CPU fp64 oracle against what the pages and the mathematics fix.

Each test ties one part of the oracle to something other than itself: a value
printed on the pages (tests/golden), a closed form, an invariant, a special
case that reduces to a library routine, or brute force on a tiny input.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import hattn_oracle as O
from full_gqa_attention_spark2_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- config
def test_layer_params_match_page_tables():
    t = _golden("spark_layer_config.json")
    for kind in ("full", "sliding"):
        p = O.layer_params(kind)
        assert p["theta"] == t["rope"][kind]["rope_theta"]
        assert p["rotary_fraction"] == t["rope"][kind]["partial_rotary_factor"]
        assert O.rotary_dim(p["rotary_fraction"]) == t["rope"][kind]["rotated_channels"]
    assert O.layer_params("sliding")["window"] == t["models"]["4B"]["sliding_window"]
    assert O.layer_params("full")["window"] is None


def test_layer_schedule_matches_page_numbering():
    t = _golden("spark_layer_config.json")
    s36 = O.layer_schedule(36)
    full_1idx = [i + 1 for i, k in enumerate(s36) if k == "full"]
    assert full_1idx == t["full_layer_numbers_1_indexed_4B"]
    assert sum(k == "full" for k in O.layer_schedule(28)) == t["models"]["1.7B"]["full_layers"]
    with pytest.raises(ValueError):
        O.layer_schedule(30)


def test_rotary_dim_rejects_non_even():
    assert O.rotary_dim(0.25) == 64
    assert O.rotary_dim(1.0) == 256
    for bad in (0.0, 0.3, 1.5, 1.0 / 256):
        with pytest.raises(ValueError):
            O.rotary_dim(bad)


# ----------------------------------------------------------------- bf16
def test_bf16_rne_matches_torch_on_fp32_values():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(200_000, generator=g) * torch.exp2(torch.randint(-140, 120, (200_000,), generator=g).float())
    ref = x.to(torch.bfloat16).double().numpy()
    got = O.bf16_rne(x.double().numpy())
    assert np.array_equal(got, ref)


def test_bf16_rne_ties_to_even_from_fp64():
    ulp = 2.0 ** -7
    # exact ties between 1 and 1+ulp go to the even mantissa (1.0), and
    # between 1+ulp and 1+2ulp to 1+2ulp
    assert O.bf16_rne(1.0 + ulp / 2) == 1.0
    assert O.bf16_rne(1.0 + 1.5 * ulp) == 1.0 + 2 * ulp
    # just above a tie rounds up: fp64 keeps bits that fp32 would drop
    assert O.bf16_rne(1.0 + ulp / 2 + 2.0 ** -40) == 1.0 + ulp
    assert O.bf16_rne(-(1.0 + ulp / 2 + 2.0 ** -40)) == -(1.0 + ulp)
    assert O.bf16_rne(0.0) == 0.0
    assert np.isinf(O.bf16_rne(3.4e38 * 1.001))


# ----------------------------------------------------------------- RoPE
@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_position_zero_is_identity(kind):
    p = O.layer_params(kind)
    x = np.random.default_rng(0).standard_normal((5, 3, 256))
    y = O.rope(x, np.zeros(5, np.int64), p["theta"], p["rotary_fraction"])
    assert np.array_equal(x, y)


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_preserves_norm_and_unrotated_channels(kind):
    p = O.layer_params(kind)
    r = O.rotary_dim(p["rotary_fraction"])
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 4, 256))
    pos = rng.integers(0, 1 << 20, size=7)
    y = O.rope(x, pos, p["theta"], p["rotary_fraction"])
    assert np.array_equal(y[..., r:], x[..., r:])
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    # each rotated pair keeps its own norm too
    h = r // 2
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:r] ** 2, x[..., :h] ** 2 + x[..., h:r] ** 2, rtol=1e-11)
    # rotating back by -p restores x
    z = O.rope(y, -pos, p["theta"], p["rotary_fraction"])
    np.testing.assert_allclose(z, x, atol=1e-11)


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_textbook_rotation_of_unit_vectors(kind):
    # rotate-half pairing: channel 0 pairs with channel r/2; frequency of
    # pair 0 is 1 whatever theta is, so at p = 1 the angle is exactly 1 rad
    p = O.layer_params(kind)
    r = O.rotary_dim(p["rotary_fraction"])
    e0 = np.zeros((1, 1, 256)); e0[..., 0] = 1.0
    y = O.rope(e0, np.array([1]), p["theta"], p["rotary_fraction"])[0, 0]
    assert y[0] == math.cos(1.0) and y[r // 2] == math.sin(1.0)
    assert np.count_nonzero(y) == 2
    eh = np.zeros((1, 1, 256)); eh[..., r // 2] = 1.0
    y = O.rope(eh, np.array([1]), p["theta"], p["rotary_fraction"])[0, 0]
    assert y[0] == -math.sin(1.0) and y[r // 2] == math.cos(1.0)


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_frequency_base_is_rotary_dim(kind):
    # inv_freq_i = theta^(-2i/r): pair r/4 turns at theta^(-1/2), and
    # successive pairs slow down by the constant factor theta^(2/r)
    p = O.layer_params(kind)
    r = O.rotary_dim(p["rotary_fraction"])
    f = O.rope_inv_freq(p["theta"], r)
    assert len(f) == r // 2 and f[0] == 1.0
    np.testing.assert_allclose(f[r // 4], 1.0 / math.sqrt(p["theta"]), rtol=1e-14)
    np.testing.assert_allclose(f[:-1] / f[1:], p["theta"] ** (2.0 / r), rtol=1e-13)


def test_rope_relative_position_property():
    # <RoPE(q, m), RoPE(k, n)> depends only on m - n
    p = O.layer_params("sliding")
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 256)); k = rng.standard_normal((1, 1, 256))
    def dot(m, n):
        a = O.rope(q, np.array([m]), p["theta"], 1.0)
        b = O.rope(k, np.array([n]), p["theta"], 1.0)
        return float((a * b).sum())
    assert abs(dot(10, 3) - dot(1007, 1000)) < 1e-10
    assert abs(dot(10, 3) - dot(3, 10)) > 1e-3


# ----------------------------------------------------------------- masks
def test_pair_count_closed_form_sliding_prefill():
    # S = 1024 queries at 0..1023 with a 512 window: sum_i min(i+1, 512)
    closed = sum(min(i + 1, 512) for i in range(1024))
    assert closed == 393_472
    assert O.pair_count(np.arange(1024), 1024, 512) == closed
    assert O.pair_count(np.arange(40), 40, 7) == sum(min(i + 1, 7) for i in range(40))
    assert O.pair_count(np.arange(40), 40, None) == 40 * 41 // 2


def test_ring_slots_by_brute_force_replay():
    for cap in (1, 5, 8):
        for n in (0, 1, cap - 1, cap, cap + 1, 3 * cap + 2):
            held = {}
            for p in range(n):
                held[p % cap] = p
            want = np.array([held.get(s, -1) for s in range(cap)])
            assert np.array_equal(O.ring_slot_positions(n, cap), want)
            assert all(O.ring_slot(p, cap) == p % cap for p in range(n))


def _small_prefill(S=37, Hq=4, Hkv=2, seed=0, q_scale=1.0, B=1):
    inp = synth.prefill_inputs(B, S, Hq, Hkv, seed=seed, q_scale=q_scale)
    return {k: O.f64(v) for k, v in inp.items()}


def test_window_covering_everything_equals_full_causal():
    x = _small_prefill()
    S = x["q"].shape[1]
    for w in (S, S + 5):
        a, _ = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], window=w, theta=1e4, rotary_fraction=1.0)
        b, _ = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], window=None, theta=1e4, rotary_fraction=1.0)
        assert np.array_equal(a, b)


def test_window_one_returns_gated_own_value():
    x = _small_prefill()
    out, _ = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [5], window=1, theta=1e4, rotary_fraction=1.0)
    G = 2
    v_self = np.repeat(x["v"], G, axis=2)
    want = v_self * O.sigmoid(x["gate"])[..., None]
    assert np.array_equal(out, want)


# ----------------------------------------------------------------- attention
@pytest.mark.parametrize("window", [None, 9])
def test_attention_matches_torch_sdpa_fp64(window):
    # library routine: scaled_dot_product_attention (default scale
    # 1/sqrt(D)), explicit boolean mask, K/V repeated for the GQA groups
    x = _small_prefill(S=29, Hq=8, Hkv=2, seed=3)
    theta, rf = 5e6, 0.25
    out, k_hat = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [100], window=window, theta=theta, rotary_fraction=rf)
    S = x["q"].shape[1]
    pos = 100 + np.arange(S)
    q_rot = O.rope(x["q"][0], pos, theta, rf)
    q_t = torch.from_numpy(q_rot).permute(1, 0, 2)                  # [Hq,S,D]
    k_t = torch.from_numpy(k_hat[0]).permute(1, 0, 2).repeat_interleave(4, 0)
    v_t = torch.from_numpy(x["v"][0]).permute(1, 0, 2).repeat_interleave(4, 0)
    i = torch.arange(S)
    mask = i[None, :] <= i[:, None]
    if window is not None:
        mask &= (i[:, None] - i[None, :]) < window
    ref = torch.nn.functional.scaled_dot_product_attention(q_t, k_t, v_t, attn_mask=mask)
    ref = ref * torch.sigmoid(torch.from_numpy(x["gate"][0]).T)[..., None]
    np.testing.assert_allclose(out[0], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_gated_mean_of_visible_values():
    x = _small_prefill(S=20, seed=4)
    x["q"][:] = 0.0
    w = 6
    out, _ = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], window=w, theta=1e4, rotary_fraction=1.0)
    for i in range(20):
        lo = max(0, i - w + 1)
        for h in range(4):
            want = x["v"][0, lo:i + 1, h // 2].mean(axis=0) * O.sigmoid(x["gate"][0, i, h])
            np.testing.assert_allclose(out[0, i, h], want, rtol=1e-13, atol=1e-15)


def test_gate_closed_forms():
    x = _small_prefill(S=16, seed=5)
    def run(gv):
        g = np.full_like(x["gate"], gv)
        return O.prefill_ref(x["q"], x["k"], x["v"], g, [0], window=None, theta=1e4, rotary_fraction=1.0)[0]
    o_half, o_one, o_34 = run(0.0), run(40.0), run(math.log(3.0))
    assert np.array_equal(o_half, 0.5 * o_one)          # sigmoid(40) == 1.0 in fp64
    np.testing.assert_allclose(o_34, 0.75 * o_one, rtol=1e-14, atol=1e-16)
    # per-head broadcast: the gated/ungated ratio is one number per (token, head)
    out = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], window=None, theta=1e4, rotary_fraction=1.0)[0]
    ratio = out / o_one
    np.testing.assert_allclose(ratio, np.broadcast_to(O.sigmoid(x["gate"])[..., None], ratio.shape), rtol=1e-12)


def test_silu_gate_closed_forms_and_library_routine():
    # the silu gate mode [SPARK §3]: silu(g) = g * sigmoid(g) in place of sigmoid(g)
    x = _small_prefill(S=16, seed=5)
    def run(gv, act):
        g = np.full_like(x["gate"], gv)
        return O.prefill_ref(x["q"], x["k"], x["v"], g, [0], window=None, theta=1e4,
                             rotary_fraction=1.0, gate_act=act)[0]
    o_one = run(40.0, "sigmoid")                        # sigmoid(40) == 1.0: ungated
    assert np.array_equal(run(0.0, "silu"), np.zeros_like(o_one))   # silu(0) = 0
    assert np.array_equal(run(40.0, "silu"), 40.0 * o_one)          # silu(40) = 40
    np.testing.assert_allclose(run(math.log(3.0), "silu"), 0.75 * math.log(3.0) * o_one,
                               rtol=1e-14, atol=1e-16)
    # per (token, head) the silu output is g times the sigmoid output
    kw = dict(window=None, theta=1e4, rotary_fraction=1.0)
    o_sig = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], **kw)[0]
    o_silu = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], gate_act="silu", **kw)[0]
    np.testing.assert_allclose(o_silu, o_sig * O.f64(x["gate"])[..., None], rtol=1e-13, atol=1e-15)
    # the gate factor itself against torch's silu in fp64, tails included
    g = np.concatenate([np.linspace(-60.0, 60.0, 2001), [-1e-300, 0.0, 1e-300]])
    want = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    np.testing.assert_allclose(O.gate_factor(g, "silu"), want, rtol=1e-15, atol=1e-300)
    with pytest.raises(ValueError):
        O.gate_factor(g, "gelu")


def test_silu_gate_in_decode_equals_prefill_row():
    # a decode step with the silu gate equals the matching prefill row
    rng = np.random.default_rng(11)
    S, Hq, Hkv, D = 9, 4, 1, 256
    q = rng.standard_normal((1, S, Hq, D))
    k = O.bf16_rne(rng.standard_normal((1, S, Hkv, D)))
    v = O.bf16_rne(rng.standard_normal((1, S, Hkv, D)))
    g = 2.0 * rng.standard_normal((1, S, Hq))
    kw = dict(window=None, theta=5e6, rotary_fraction=0.25, gate_act="silu")
    pre, k_hat = O.prefill_ref(q, k, v, g, [0], **kw)
    cap = 16
    ck = np.zeros((1, Hkv, cap, D))
    cv = np.zeros((1, Hkv, cap, D))
    ck[0, :, :S - 1] = k_hat[0, :S - 1].transpose(1, 0, 2)
    cv[0, :, :S - 1] = v[0, :S - 1].transpose(1, 0, 2)
    dec, _, _ = O.decode_ref(q[:, S - 1], k[:, S - 1], v[:, S - 1], g[:, S - 1], [S - 1], ck, cv,
                             kind="linear", **kw)
    np.testing.assert_allclose(dec[0], pre[0, S - 1], rtol=1e-12, atol=1e-14)


def test_varlen_prefill_equal_lengths_is_the_uniform_batch():
    x = _small_prefill(S=12, seed=21, B=3)
    kw = dict(window=5, theta=1e4, rotary_fraction=1.0)
    out, kh = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0, 7, 30], **kw)
    pk = lambda t: O.f64(t).reshape((-1,) + tuple(t.shape[2:]))
    vo, vk = O.prefill_varlen_ref(pk(x["q"]), pk(x["k"]), pk(x["v"]), pk(x["gate"]), [0, 12, 24, 36],
                                  [0, 7, 30], **kw)
    assert np.array_equal(vo, out.reshape(vo.shape)) and np.array_equal(vk, kh.reshape(vk.shape))


def test_varlen_prefill_sequences_are_independent():
    # ragged lengths (one empty): each sequence's rows equal a batch of one,
    # whatever the others hold, and the empty one produces nothing
    rng = np.random.default_rng(22)
    lens, starts = [5, 0, 9, 1], [3, 11, 0, 40]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((T, 8, 256))
    k = O.bf16_rne(rng.standard_normal((T, 2, 256)))
    v = O.bf16_rne(rng.standard_normal((T, 2, 256)))
    g = 2.0 * rng.standard_normal((T, 8))
    hk = O.bf16_rne(rng.standard_normal((4, 2, 64, 256)))
    hv = O.bf16_rne(rng.standard_normal((4, 2, 64, 256)))
    hp = np.stack([O.linear_slot_positions(s, 64) for s in starts])
    kw = dict(window=None, theta=5e6, rotary_fraction=0.25)
    out, kh = O.prefill_varlen_ref(q, k, v, g, cu, starts, hist_k=hk, hist_v=hv, hist_pos=hp, **kw)
    for b in range(4):
        lo, hi = cu[b], cu[b + 1]
        if hi == lo:
            continue
        o1, k1 = O.prefill_ref(q[None, lo:hi], k[None, lo:hi], v[None, lo:hi], g[None, lo:hi], [starts[b]],
                               hist_k=hk[b:b + 1], hist_v=hv[b:b + 1], hist_pos=hp[b:b + 1], **kw)
        assert np.array_equal(out[lo:hi], o1[0]) and np.array_equal(kh[lo:hi], k1[0])
    # changing another sequence's tokens leaves sequence 2 unchanged
    q2 = q.copy()
    q2[:cu[2]] += 1.0
    out2, _ = O.prefill_varlen_ref(q2, k, v, g, cu, starts, hist_k=hk, hist_v=hv, hist_pos=hp, **kw)
    assert np.array_equal(out2[cu[2]:cu[3]], out[cu[2]:cu[3]])
    with pytest.raises(ValueError):
        O.prefill_varlen_ref(q, k, v, g, [0, 5, 4, 15, 15], starts, **kw)


def test_paged_to_linear_by_brute_force():
    # every slot of every sequence, looked up one by one
    rng = np.random.default_rng(23)
    B, Hkv, ps, n = 3, 2, 4, 5
    pool = rng.standard_normal((B * n + 2, Hkv, ps, 3))
    table = rng.permutation(B * n + 2)[:B * n].reshape(B, n)
    lin = O.paged_to_linear(pool, table, ps)
    assert lin.shape == (B, Hkv, n * ps, 3)
    for b in range(B):
        for p in range(n * ps):
            assert np.array_equal(lin[b, :, p], pool[table[b, p // ps], :, p % ps])


def test_new_keys_are_cached_as_bf16():
    x = _small_prefill(S=12, seed=6)
    _, kh = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [77], window=None, theta=5e6, rotary_fraction=0.25)
    _, kp = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [77], window=None, theta=5e6, rotary_fraction=0.25, round_keys=False)
    assert np.array_equal(O.bf16_rne(kh), kh)
    assert not np.array_equal(kh, kp)
    assert np.max(np.abs(kh - kp)) <= np.max(np.abs(kp)) * 2.0 ** -8


def test_shift_invariance_of_pure_variant():
    # relative RoPE: moving every position by the same amount changes nothing
    x = _small_prefill(S=25, seed=7)
    a, _ = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], window=8, theta=1e4, rotary_fraction=1.0, round_keys=False)
    b, _ = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [123457], window=8, theta=1e4, rotary_fraction=1.0, round_keys=False)
    np.testing.assert_allclose(a, b, atol=1e-9)


# ----------------------------------------------------------------- caches
def test_chunked_prefill_equals_monolithic():
    x = _small_prefill(S=40, seed=8)
    kw = dict(window=11, theta=1e4, rotary_fraction=1.0)
    full, kh = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], **kw)
    c = 23
    first, kh1 = O.prefill_ref(x["q"][:, :c], x["k"][:, :c], x["v"][:, :c], x["gate"][:, :c], [0], **kw)
    hist_k = kh1.transpose(0, 2, 1, 3)
    hist_v = x["v"][:, :c].transpose(0, 2, 1, 3)
    second, _ = O.prefill_ref(x["q"][:, c:], x["k"][:, c:], x["v"][:, c:], x["gate"][:, c:], [c],
                              hist_k=hist_k, hist_v=hist_v, hist_pos=np.arange(c)[None], **kw)
    np.testing.assert_allclose(np.concatenate([first, second], axis=1), full, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("kind", ["ring", "linear"])
def test_decode_equals_prefill_row(kind):
    S, w = 30, 8
    x = _small_prefill(S=S, seed=9)
    kw = dict(window=w, theta=1e4, rotary_fraction=1.0)
    full, kh = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], **kw)
    p = S - 1
    cap = w if kind == "ring" else S + 3
    ck = np.zeros((1, 2, cap, 256)); cv = np.zeros((1, 2, cap, 256))
    for t in range(p):  # replay writes of positions 0..p-1
        s = t % cap if kind == "ring" else t
        ck[0, :, s] = kh[0, t]; cv[0, :, s] = x["v"][0, t]
    out, slots, k_hat = O.decode_ref(x["q"][:, p], x["k"][:, p], x["v"][:, p], x["gate"][:, p], [p],
                                     ck, cv, kind=kind, **kw)
    assert slots[0] == (p % cap if kind == "ring" else p)
    assert np.array_equal(k_hat[0], kh[0, p])
    np.testing.assert_allclose(out[0], full[0, p], rtol=1e-13, atol=1e-15)


def test_ring_decode_with_partial_ring():
    # positions below w-1: only slots 0..p hold tokens
    S, w = 5, 8
    x = _small_prefill(S=S, seed=10)
    kw = dict(window=w, theta=1e4, rotary_fraction=1.0)
    full, kh = O.prefill_ref(x["q"], x["k"], x["v"], x["gate"], [0], **kw)
    ck = np.full((1, 2, w, 256), 1e3); cv = np.full((1, 2, w, 256), 1e3)  # junk in unwritten slots
    p = 4
    ck[0, :, :p] = kh[0, :p].transpose(1, 0, 2); cv[0, :, :p] = x["v"][0, :p].transpose(1, 0, 2)
    out, _, _ = O.decode_ref(x["q"][:, p], x["k"][:, p], x["v"][:, p], x["gate"][:, p], [p], ck, cv, kind="ring", **kw)
    np.testing.assert_allclose(out[0], full[0, p], rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------- sizing
def test_kv_sizing_matches_page_table():
    t = _golden("kv_cache_sizing.json")
    assert O.kv_bytes_per_token_layer(4) == t["bytes_per_token_per_layer_4B"]
    assert O.kv_bytes_per_token_layer(2) == t["bytes_per_token_per_layer_1_7B"]
    T = t["tokens"]
    for row in t["rows"]:
        n, h = row["n_layers"], row["kv_heads"]
        per = O.kv_bytes_per_token_layer(h)
        sched = O.layer_schedule(n)
        if row["part"] == "full":
            got = sum(T * per for k in sched if k == "full")
        elif row["part"] == "sliding":
            got = sum(min(T, 512) * per for k in sched if k == "sliding")
        else:
            got = O.kv_bytes_model(n, h, T, hybrid=False)
        assert abs(got / row["page_value_bytes"] - 1) <= row["rel_tol"], row["what"]
    ratio = O.kv_bytes_model(36, 4, T) / O.kv_bytes_model(36, 4, T, hybrid=False)
    assert abs(ratio - t["ratio_hybrid_over_all_full"]) <= t["ratio_rel_tol"]
    assert O.kv_bytes_model(36, 4, 1 << 20, hybrid=False) == t["all_full_2pow20_GiB_explainer_page"] * 2 ** 30


# ----------------------------------------------------------------- the attention block
def _block_case(T=9, H=64, Hq=4, Hkv=1, seed=31):
    rng = np.random.default_rng(seed)
    D = 256
    x = O.bf16_rne(rng.standard_normal((T, H)))
    nw = O.bf16_rne(1.0 + 0.1 * rng.standard_normal(H))
    wq = O.bf16_rne(0.05 * rng.standard_normal(((Hq + 2 * Hkv) * D + Hq, H)))
    wo = O.bf16_rne(0.02 * rng.standard_normal((H, Hq * D)))
    return x, nw, wq, wo


def test_rms_norm_against_torch_and_closed_form():
    rng = np.random.default_rng(32)
    x = O.bf16_rne(rng.standard_normal((7, 96)))
    w = O.bf16_rne(1.0 + 0.1 * rng.standard_normal(96))
    got = O.rms_norm(x, w, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), 1e-6).numpy()
    # one bf16 rounding of the library's fp64 result: within half an ulp of it
    half_ulp = 2.0 ** (np.floor(np.log2(np.abs(ref))) - 8)
    assert np.all(np.abs(got - ref) <= half_ulp * (1 + 1e-12))
    # a constant row c: every channel becomes w * c / sqrt(c^2 + eps)
    c, eps = -1.5, 1e-6
    got = O.rms_norm(np.full((1, 96), c), w, eps)
    assert np.array_equal(got[0], O.bf16_rne(w * c / math.sqrt(c * c + eps)))


def test_block_with_zero_out_proj_returns_the_residual():
    x, nw, wq, _ = _block_case()
    wo = np.zeros((x.shape[1], 4 * 256))
    out, _ = O.block_prefill_ref(x, nw, wq, wo, 1e-6, [0, x.shape[0]], [0], Hq=4, Hkv=1, window=None,
                                 theta=5e6, rotary_fraction=0.25)
    assert np.array_equal(out, x)


def test_block_projection_orientation_and_split_order():
    # out_proj as a permutation matrix: y[:, i] = attn[:, sigma(i)]; the
    # fused projection rows pick normed channels, so q/k/v/g are known slices
    T, H, Hq, Hkv, D = 6, 4 * 256, 4, 1, 256
    rng = np.random.default_rng(33)
    x = O.bf16_rne(rng.standard_normal((T, H)))
    nw = np.ones(H)
    tau = rng.integers(0, H, (Hq + 2 * Hkv) * D + Hq)
    wq = np.zeros((tau.size, H))
    wq[np.arange(tau.size), tau] = 1.0
    sigma = rng.permutation(Hq * D)
    wo = np.zeros((H, Hq * D))
    wo[np.arange(H), sigma] = 1.0
    kw = dict(window=None, theta=5e6, rotary_fraction=0.25)
    out, _ = O.block_prefill_ref(x, nw, wq, wo, 1e-6, [0, T], [3], Hq=Hq, Hkv=Hkv, **kw)
    h = O.rms_norm(x, nw, 1e-6)[:, tau]
    q = h[:, :Hq * D].reshape(T, Hq, D)
    k = h[:, Hq * D:(Hq + 1) * D].reshape(T, 1, D)
    v = h[:, (Hq + 1) * D:(Hq + 2) * D].reshape(T, 1, D)
    g = h[:, (Hq + 2) * D:]
    attn, _ = O.prefill_varlen_ref(q, k, v, g, [0, T], [3], **kw)
    assert np.array_equal(out, x + O.bf16_rne(attn).reshape(T, -1)[:, sigma])


def test_block_decode_equals_block_prefill_row():
    x, nw, wq, wo = _block_case(T=9)
    kw = dict(Hq=4, Hkv=1, window=None, theta=5e6, rotary_fraction=0.25, gate_act="sigmoid")
    full, k_hat = O.block_prefill_ref(x, nw, wq, wo, 1e-6, [0, 9], [0], **kw)
    h = O.rms_norm(x[:8], nw, 1e-6)
    _, _, v8, _ = O.split_qkvg(O.linear_bf16(h, wq), 4, 1)
    ck = np.zeros((1, 1, 16, 256))
    cv = np.zeros((1, 1, 16, 256))
    ck[0, 0, :8] = k_hat[:8, 0]
    cv[0, 0, :8] = v8[:, 0]
    kd = dict(kw)
    kd.pop("window")
    dec, _, _ = O.block_decode_ref(x[8:9], nw, wq, wo, 1e-6, [8], ck, cv, kind="linear", window=None, **kd)
    np.testing.assert_allclose(dec[0], full[8], rtol=0, atol=1e-12)
