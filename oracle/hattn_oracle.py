"""CPU fp64 oracle for the hybrid sliding-window / full causal GQA attention core.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (the HIP library and its Python binding) never touches it, and
this module imports nothing from the product path: the two share no code,
tables or constants.

What it computes is the plain definition, written out in fp64 numpy (a matmul,
``exp``, ``cos``/``sin`` are the only library primitives used):

  out = softmax(RoPE(q) . K_hat^T / sqrt(d_head) + mask) V  *  sigmoid(g)

Sources, cited by page title and section:

* [SPARK] "Spark-X2.5 架构（4B / 1.7B）": §1 config table, §2 hybrid attention
  (mask per layer type), §3 head-wise output gate and its Eq. 1, §4 layered
  RoPE table, §6 KV-cache sizing table.
* [EXPL] "Spark-X2.5-4B混合注意力架构原理…" (one long section): the sliding
  layers keep only the 512 most recent tokens in their KV cache; the cache is
  written by ``past_key_values.update`` inside the attention forward.
* [PROPE] the architecture-survey page, §13.3 "部分旋转位置编码（Partial RoPE）":
  with partial RoPE only the first ``rotary_dim`` channels of each head are
  rotated and the rest pass through unchanged.

Readings taken where the pages are silent (each is repeated where it is used):

* window: a query at p_q sees a key at p_k iff p_k <= p_q and p_q - p_k < w,
  i.e. itself plus the w-1 previous tokens; a 512-slot ring then holds exactly
  the visible set.
* the new token's K/V are written to the cache before attention reads it, so
  the cache stores the rotated key rounded once to bf16 (K_hat) and V as given;
  Q, scores, probabilities and the output stay fp64.
* RoPE pairs channel i with channel i + r/2 (rotate-half) inside the first r
  channels, r = head_dim * rotary_fraction, with inv_freq_i = theta^(-2i/r);
  the angle p * inv_freq_i is formed in fp64. The pairing convention itself is
  not fixed by the pages (parity unpinned for the pairing; the rotated set and
  the frequency base are).
* GQA: q-head h reads kv-head h // (Hq / Hkv).
* Scale 1/sqrt(256) = 1/16, no softcap, no q/k norm.
* The gate is sigmoid of one logit per (token, head), broadcast over the
  head's channels; the oracle's output is the unrounded fp64 product. [SPARK
  §3] also notes that the model code accepts a silu gate activation; it is
  read as silu(g) = g * sigmoid(g) in place of sigmoid(g), nothing else
  changed.
* Ring slot of position p is p mod capacity; a ring requires capacity == w.
"""
from __future__ import annotations

import math

import numpy as np

try:  # torch is only used to read bf16 tensors; the arithmetic is numpy
    import torch as _torch
except Exception:  # pragma: no cover
    _torch = None

HEAD_DIM = 256
SCALE = 1.0 / math.sqrt(HEAD_DIM)


# --------------------------------------------------------------------------
# layer configuration  [SPARK §1 config table, §2, §4 RoPE table]
# --------------------------------------------------------------------------
def layer_params(layer_type: str) -> dict:
    """Per-layer-type attention parameters as the pages state them.

    [SPARK §4 table]: full_attention uses rope_theta 5e6 and
    partial_rotary_factor 0.25 (first 64 of 256 channels); sliding_attention
    uses rope_theta 1e4 and factor 1.0 (all 256 channels).
    [SPARK §1 table, §2]: sliding layers get sliding_window = 512, full layers
    get no window (None = unbounded causal).
    """
    if layer_type == "sliding":
        return {"window": 512, "theta": 1.0e4, "rotary_fraction": 1.0}
    if layer_type == "full":
        return {"window": None, "theta": 5.0e6, "rotary_fraction": 0.25}
    raise ValueError(f"unknown layer type {layer_type!r}")


def layer_schedule(n_layers: int) -> list:
    """[SPARK §1 table, §2]: layer_types is (sliding, sliding, sliding, full)
    repeated; 36 layers (4B) or 28 layers (1.7B)."""
    if n_layers <= 0 or n_layers % 4:
        raise ValueError("layer count must be a positive multiple of 4")
    return ["full" if i % 4 == 3 else "sliding" for i in range(n_layers)]


def rotary_dim(rotary_fraction: float, head_dim: int = HEAD_DIM) -> int:
    """Number of rotated channels r = head_dim * fraction [SPARK §4 table].
    Must be a positive even integer no larger than head_dim."""
    r = rotary_fraction * head_dim
    if r <= 0 or r > head_dim or r != int(r) or int(r) % 2:
        raise ValueError(f"rotary_fraction {rotary_fraction} gives r={r}")
    return int(r)


# --------------------------------------------------------------------------
# numeric helpers
# --------------------------------------------------------------------------
def f64(x) -> np.ndarray:
    """Exact conversion of a numpy array or a CPU torch tensor (bf16/fp32) to
    an fp64 numpy array."""
    if _torch is not None and isinstance(x, _torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def bf16_rne(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even, directly
    from fp64 (no intermediate fp32 rounding). bfloat16 keeps 8 significant
    bits and the fp32 exponent range; below 2^-126 the spacing is 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    m, e = np.frexp(x[fin])                       # x = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # 8 significant bits, RNE
    small = np.abs(x[fin]) < 2.0 ** -126
    r[small] = np.ldexp(np.rint(np.ldexp(x[fin][small], 133)), -133)
    big = np.abs(r) > (2.0 - 2.0 ** -7) * 2.0 ** 127
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    out[~fin] = x[~fin]
    return out


def sigmoid(g) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-g))


GATE_ACTS = ("sigmoid", "silu")


def gate_factor(g, gate_act: str = "sigmoid") -> np.ndarray:
    """The per-head output gate [SPARK §3 Eq. 1]: sigmoid(g); or, for the
    silu gate mode the section mentions, silu(g) = g * sigmoid(g)."""
    if gate_act == "sigmoid":
        return sigmoid(g)
    if gate_act == "silu":
        g = np.asarray(g, dtype=np.float64)
        return g * sigmoid(g)
    raise ValueError(f"unknown gate activation {gate_act!r}")


# --------------------------------------------------------------------------
# RoPE  [SPARK §4 table and text; PROPE §13.3]
# --------------------------------------------------------------------------
def rope_inv_freq(theta: float, r: int) -> np.ndarray:
    """inv_freq_i = theta^(-2i/r), i in [0, r/2), fp64. The base of the
    partial rotation is r (64 on full layers), not head_dim."""
    i = np.arange(r // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / r)


def rope(x, pos, theta: float, rotary_fraction: float) -> np.ndarray:
    """Rotate the first r channels of every head of x by the token's position.

    x: [..., T, H, D] (fp64-convertible), pos: [..., T] integer positions.
    Channel pair (i, i + r/2), i < r/2, is rotated by the angle
    pos * inv_freq_i; channels r..D-1 are returned unchanged [PROPE §13.3].
    """
    x = np.array(f64(x), dtype=np.float64, copy=True)
    r = rotary_dim(rotary_fraction, x.shape[-1])
    h = r // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(theta, r)
    c = np.cos(ang)[..., None, :]          # [..., T, 1, h]: shared by all heads
    s = np.sin(ang)[..., None, :]
    a = x[..., :h].copy()
    b = x[..., h:r].copy()
    x[..., :h] = a * c - b * s
    x[..., h:r] = b * c + a * s
    return x


# --------------------------------------------------------------------------
# masks and cache slots  [SPARK §2; EXPL sliding-layer cache paragraph]
# --------------------------------------------------------------------------
def allowed(p_q, p_k, window) -> np.ndarray:
    """Causal (and, for sliding layers, windowed) visibility of key position
    p_k from query position p_q. Negative p_k marks an empty slot."""
    p_q = np.asarray(p_q, dtype=np.int64)
    p_k = np.asarray(p_k, dtype=np.int64)
    ok = (p_k >= 0) & (p_k <= p_q)
    if window is not None:
        ok &= (p_q - p_k) < int(window)
    return ok


def ring_slot(p, capacity: int):
    """Slot that position p is written to in a ring of the given capacity."""
    return np.asarray(p, dtype=np.int64) % int(capacity)


def ring_slot_positions(next_pos: int, capacity: int) -> np.ndarray:
    """Position held by each ring slot after positions 0..next_pos-1 have
    been written in order (slot s keeps the largest such position that is
    congruent to s); -1 for a slot never written."""
    s = np.arange(capacity, dtype=np.int64)
    last = int(next_pos) - 1
    p = last - np.mod(last - s, capacity)
    p[p < 0] = -1
    return p


def linear_slot_positions(next_pos: int, capacity: int) -> np.ndarray:
    """Position held by each linear-cache slot after positions
    0..next_pos-1 were written (slot == position); -1 if not yet written."""
    s = np.arange(capacity, dtype=np.int64)
    return np.where(s < int(next_pos), s, -1)


# --------------------------------------------------------------------------
# attention  [SPARK §3 Eq. 1]
# --------------------------------------------------------------------------
def attend(q_rot, keys, values, ok, gate_logit, gate_act="sigmoid") -> np.ndarray:
    """Gated softmax attention of query rows against one kv-head's keys.

    q_rot: [M, D] rotated queries, keys/values: [N, D], ok: [M, N] visibility,
    gate_logit: [M]. Returns [M, D] fp64:
      softmax(q k^T / sqrt(D) over visible keys) V * sigmoid(g)   (Eq. 1),
    with silu(g) in place of sigmoid(g) for gate_act="silu".
    """
    q_rot = f64(q_rot)
    keys = f64(keys)
    values = f64(values)
    ok = np.asarray(ok, dtype=bool)
    if not ok.any(axis=1).all():
        raise ValueError("a query row sees no key")
    s = (q_rot @ keys.T) * SCALE
    s = np.where(ok, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    a = e / e.sum(axis=1, keepdims=True)
    o = a @ values
    return o * gate_factor(gate_logit, gate_act)[:, None]


def prefill_ref(q, k, v, gate, start_pos, *, window, theta, rotary_fraction,
                hist_k=None, hist_v=None, hist_pos=None, rows=None,
                round_keys=True, gate_act="sigmoid"):
    """One prefill call: S new tokens per sequence at positions
    start_pos[b] + 0..S-1, attending to the cached history plus themselves.

    q: [B, S, Hq, D], k/v: [B, S, Hkv, D], gate: [B, S, Hq].
    hist_k/hist_v: [B, Hkv, Nh, D] cached (already rotated, bf16-valued) keys
    and values; hist_pos: [B, Nh] their positions (-1 = empty slot).
    rows: optional sorted indices into S; only those query rows are computed.
    round_keys: store the rotated new keys as bf16 before use (the cache
    holds bf16, [SPARK §1 dtype, §6]); False gives the pure fp64 variant.
    gate_act: "sigmoid" (Eq. 1) or "silu" (the alternative gate mode).

    Returns (out [B, len(rows), Hq, D] fp64, k_hat [B, S, Hkv, D] fp64):
    k_hat is what the call writes to the cache for the new keys.
    """
    q = f64(q)
    k = f64(k)
    v = f64(v)
    gate = f64(gate)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, len(rows), Hq, D))
    k_hat_all = np.zeros((B, S, Hkv, D))
    for b in range(B):
        pos = int(start_pos[b]) + np.arange(S, dtype=np.int64)
        q_rot = rope(q[b], pos, theta, rotary_fraction)          # [S, Hq, D]
        k_rot = rope(k[b], pos, theta, rotary_fraction)          # [S, Hkv, D]
        k_hat = bf16_rne(k_rot) if round_keys else k_rot
        k_hat_all[b] = k_hat
        if hist_k is not None:
            key_pos = np.concatenate([np.asarray(hist_pos[b], np.int64), pos])
        else:
            key_pos = pos
        ok = allowed(pos[rows][:, None], key_pos[None, :], window)
        for g in range(Hkv):
            keys = k_hat[:, g]
            vals = v[b, :, g]
            if hist_k is not None:
                keys = np.concatenate([f64(hist_k[b, g]), keys])
                vals = np.concatenate([f64(hist_v[b, g]), vals])
            for h in range(g * G, (g + 1) * G):
                out[b, :, h] = attend(q_rot[rows, h], keys, vals, ok,
                                      gate[b, rows, h], gate_act)
    return out, k_hat_all


def prefill_varlen_ref(q, k, v, gate, cu_seqlens, start_pos, *, window, theta,
                       rotary_fraction, hist_k=None, hist_v=None, hist_pos=None,
                       round_keys=True, gate_act="sigmoid"):
    """A ragged batch of prefills: sequence b's new tokens are the packed
    rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of q [T, Hq, D], k/v [T, Hkv, D]
    and gate [T, Hq], at positions start_pos[b] + 0, 1, ...; each sequence
    is its own prefill_ref call over its own history (hist_* indexed by b as
    in prefill_ref). Returns (out [T, Hq, D], k_hat [T, Hkv, D]) in packed
    order."""
    q = f64(q)
    k = f64(k)
    v = f64(v)
    gate = f64(gate)
    cu = [int(x) for x in cu_seqlens]
    T = q.shape[0]
    if cu[0] != 0 or cu[-1] != T or any(b > a for a, b in zip(cu[1:], cu[:-1])):
        raise ValueError("cu_seqlens must start at 0, not decrease and end at T")
    out = np.zeros(q.shape)
    k_hat = np.zeros(k.shape)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        if hi == lo:
            continue
        hist = {}
        if hist_k is not None:
            hist = dict(hist_k=hist_k[b:b + 1], hist_v=hist_v[b:b + 1], hist_pos=hist_pos[b:b + 1])
        o, kh = prefill_ref(q[None, lo:hi], k[None, lo:hi], v[None, lo:hi], gate[None, lo:hi],
                            [start_pos[b]], window=window, theta=theta,
                            rotary_fraction=rotary_fraction, round_keys=round_keys,
                            gate_act=gate_act, **hist)
        out[lo:hi] = o[0]
        k_hat[lo:hi] = kh[0]
    return out, k_hat


def decode_ref(q, k, v, gate, pos, cache_k, cache_v, *, kind, window, theta,
               rotary_fraction, round_keys=True, gate_act="sigmoid"):
    """One decode step: one new token per sequence at position pos[b].

    q: [B, Hq, D], k/v: [B, Hkv, D], gate: [B, Hq]; cache_k/cache_v:
    [B, Hkv, cap, D] (numpy or CPU torch, bf16 values) holding positions
    0..pos[b]-1 as ``kind`` ("ring" or "linear") lays them out.
    The new key is rotated, rounded to bf16 and written at its slot
    (p mod cap for a ring, p for a linear cache) before attention reads the
    cache. Returns (out [B, Hq, D] fp64, slots [B], k_hat [B, Hkv, D]).
    The cache arguments are not modified.
    """
    q = f64(q)
    k = f64(k)
    v = f64(v)
    gate = f64(gate)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    cap = cache_k.shape[2]
    if kind == "ring" and window != cap:
        raise ValueError("a ring cache needs capacity == window")
    out = np.zeros((B, Hq, D))
    slots = np.zeros(B, dtype=np.int64)
    k_hats = np.zeros((B, Hkv, D))
    for b in range(B):
        p = int(pos[b])
        q_rot = rope(q[b][None], np.array([p]), theta, rotary_fraction)[0]
        k_rot = rope(k[b][None], np.array([p]), theta, rotary_fraction)[0]
        k_hat = bf16_rne(k_rot) if round_keys else k_rot
        k_hats[b] = k_hat
        if kind == "ring":
            slot = int(ring_slot(p, cap))
            key_pos = ring_slot_positions(p + 1, cap)
        elif kind == "linear":
            if p >= cap:
                raise ValueError("position beyond linear capacity")
            slot = p
            key_pos = linear_slot_positions(p + 1, cap)
        else:
            raise ValueError(kind)
        slots[b] = slot
        ok = allowed(p, key_pos, window)
        idx = np.nonzero(ok)[0]
        for g in range(Hkv):
            keys = f64(cache_k[b, g][idx])
            vals = f64(cache_v[b, g][idx])
            at = np.nonzero(idx == slot)[0]
            keys[at] = k_hat[g]
            vals[at] = v[b, g]
            for h in range(g * G, (g + 1) * G):
                out[b, h] = attend(q_rot[h][None], keys, vals,
                                   np.ones((1, len(idx)), bool),
                                   gate[b, h:h + 1], gate_act)[0]
    return out, slots, k_hats


# --------------------------------------------------------------------------
# the attention block around the core  [SPARK §2 figure 1 (decoder-layer
# dataflow), §1 config table, §3, §5]
# --------------------------------------------------------------------------
def rms_norm(x, weight, eps):
    """[SPARK §5] RMSNorm: computed in higher precision (fp64 here; the page
    says the model upcasts to fp32), multiplied by the weight, then cast
    back to the model dtype (bf16, one rounding)."""
    x = f64(x)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return bf16_rne(x * r * f64(weight))


def linear_bf16(x, w):
    """A bias-free Linear of the model ([SPARK §5]: attention_bias false):
    x [..., in] @ w[out, in]^T in fp64, output cast to bf16."""
    return bf16_rne(f64(x) @ f64(w).T)


def split_qkvg(y, Hq, Hkv, D=HEAD_DIM):
    """The fused projection's output [T, Hq*D + 2*Hkv*D + Hq] split into
    q [T, Hq, D], k and v [T, Hkv, D] (q_k_v_proj, [SPARK §3]: 4096 + 2 x
    1024 outputs on the 4B shape, read as Q then K then V) and the gate
    logits [T, Hq] (g_proj, one per head)."""
    T = y.shape[0]
    q = y[:, :Hq * D].reshape(T, Hq, D)
    k = y[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    v = y[:, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(T, Hkv, D)
    g = y[:, (Hq + 2 * Hkv) * D:]
    if g.shape[1] != Hq:
        raise ValueError("fused projection width does not match the head counts")
    return q, k, v, g


def block_prefill_ref(x, norm_w, w_qkvg, w_o, eps, cu_seqlens, start_pos, *, Hq, Hkv,
                      window, theta, rotary_fraction, gate_act="sigmoid", hist_k=None,
                      hist_v=None, hist_pos=None):
    """One attention block over a ragged batch of new tokens x [T, hidden]
    ([SPARK] figure 1): RMSNorm -> fused q/k/v/g projection -> the core
    (prefill_varlen_ref) -> out_proj -> + residual. x is the residual
    stream, which [SPARK §5] keeps in fp32 (the input embedding is taken to
    fp32 for the backbone); module outputs are bf16 (the model dtype; the
    core's output is cast back as [SPARK §3] states); the returned sum
    x + out_proj(...) is left unrounded.
    Returns (out [T, hidden] fp64, k_hat [T, Hkv, D])."""
    h = rms_norm(x, norm_w, eps)
    q, k, v, g = split_qkvg(linear_bf16(h, w_qkvg), Hq, Hkv)
    attn, k_hat = prefill_varlen_ref(q, k, v, g, cu_seqlens, start_pos, window=window, theta=theta,
                                     rotary_fraction=rotary_fraction, hist_k=hist_k, hist_v=hist_v,
                                     hist_pos=hist_pos, gate_act=gate_act)
    y = linear_bf16(bf16_rne(attn).reshape(attn.shape[0], -1), w_o)
    return f64(x) + y, k_hat


def block_decode_ref(x, norm_w, w_qkvg, w_o, eps, pos, cache_k, cache_v, *, Hq, Hkv, kind,
                     window, theta, rotary_fraction, gate_act="sigmoid"):
    """The block for one new token per sequence, x [B, hidden], over the
    caches as decode_ref reads them. Returns (out [B, hidden] fp64 unrounded,
    slots, k_hat)."""
    h = rms_norm(x, norm_w, eps)
    q, k, v, g = split_qkvg(linear_bf16(h, w_qkvg), Hq, Hkv)
    attn, slots, k_hat = decode_ref(q, k, v, g, pos, cache_k, cache_v, kind=kind, window=window,
                                    theta=theta, rotary_fraction=rotary_fraction, gate_act=gate_act)
    y = linear_bf16(bf16_rne(attn).reshape(attn.shape[0], -1), w_o)
    return f64(x) + y, slots, k_hat


def paged_to_linear(pool, table, page_size):
    """The linear view [B, Hkv, pages_per_seq * page_size, D] of a paged
    cache: pool [num_pages, Hkv, page_size, D], table [B, pages_per_seq];
    slot p of sequence b is row p % page_size of page table[b, p //
    page_size] (the layout the library documents for a paged cache, which
    the pages leave to the implementation)."""
    pool = np.asarray(pool)
    table = np.asarray(table)
    B, n = table.shape
    out = np.zeros((B, pool.shape[1], n * page_size) + pool.shape[3:], dtype=pool.dtype)
    for b in range(B):
        for i in range(n):
            out[b, :, i * page_size:(i + 1) * page_size] = pool[table[b, i]]
    return out


# --------------------------------------------------------------------------
# KV-cache sizing  [SPARK §6 KV table]
# --------------------------------------------------------------------------
def kv_bytes_per_token_layer(num_kv_heads: int, head_dim: int = HEAD_DIM,
                             dtype_bytes: int = 2) -> int:
    """K and V, each num_kv_heads x head_dim values of dtype_bytes."""
    return 2 * num_kv_heads * head_dim * dtype_bytes


def kv_bytes_model(n_layers: int, num_kv_heads: int, tokens: int,
                   window: int = 512, hybrid: bool = True) -> int:
    """Total KV bytes of a model at a context of ``tokens``: full layers keep
    every token, sliding layers at most ``window`` tokens. hybrid=False
    prices every layer as a full layer."""
    per = kv_bytes_per_token_layer(num_kv_heads)
    total = 0
    for t in layer_schedule(n_layers):
        kept = tokens if (t == "full" or not hybrid) else min(tokens, window)
        total += kept * per
    return total


def pair_count(q_pos, n_keys_pos, window) -> int:
    """Number of visible (query, key) pairs for queries at q_pos over keys
    at positions 0..n_keys_pos-1 (brute force)."""
    kp = np.arange(n_keys_pos, dtype=np.int64)
    return int(sum(int(allowed(p, kp, window).sum()) for p in np.asarray(q_pos)))
