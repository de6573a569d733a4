"""Seeded synthetic inputs shared by the tests, the bench and the CPU checker.

This module holds no attention arithmetic: it only draws numbers. Everything
is drawn on the CPU with ``torch.Generator`` in fp32 and rounded to bf16
(round-to-nearest-even, torch's conversion), so every consumer sees the same
bits whatever device it later copies them to.

Draw order inside one call: Q, K, V, gate logits. Caches and positions come
from their own calls with their own seeds. Large caches are drawn in chunks,
chunk c from a PCG64 generator seeded with (seed, c), in parallel threads; the
content does not depend on the thread count.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

GATE_STD = 2.0  # gate logits ~ N(0, std 2)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _normal(gen, shape, std=1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def prefill_inputs(B, S, Hq, Hkv, D=256, seed=0, q_scale=1.0):
    """Q [B,S,Hq,D], K/V [B,S,Hkv,D] ~ N(0,1); gate logits [B,S,Hq] ~ N(0, 2^2).
    q_scale multiplies the standard deviation of Q (peaky-softmax cases)."""
    g = _gen(seed)
    q = _normal(g, (B, S, Hq, D), q_scale)
    k = _normal(g, (B, S, Hkv, D))
    v = _normal(g, (B, S, Hkv, D))
    gate = _normal(g, (B, S, Hq), GATE_STD)
    return {"q": q, "k": k, "v": v, "gate": gate}


def decode_inputs(B, Hq, Hkv, D=256, seed=0):
    """q [B,Hq,D], new k/v [B,Hkv,D] ~ N(0,1); gate logits [B,Hq] ~ N(0, 2^2)."""
    g = _gen(seed)
    q = _normal(g, (B, Hq, D))
    k = _normal(g, (B, Hkv, D))
    v = _normal(g, (B, Hkv, D))
    gate = _normal(g, (B, Hq), GATE_STD)
    return {"q": q, "k": k, "v": v, "gate": gate}


def _cache_chunk(seed, c, n):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(c)])))
    return torch.from_numpy(rng.standard_normal(n, dtype=np.float32)).to(torch.bfloat16)


def cache_tensor(B, Hkv, cap, D=256, seed=0, fill_tokens=None,
                 chunk_tokens=1 << 14, out=None, threads=8):
    """bf16 cache [B, Hkv, cap, D] ~ N(0,1), drawn chunk by chunk along the
    token axis: chunk c (counting over b, head, token blocks) comes from a
    PCG64 generator seeded with (seed, c), so chunks can be drawn in
    parallel and the result does not depend on the thread count. Only the
    first ``fill_tokens`` slots of every (b, head) are drawn (default: all);
    the rest are zero. ``out`` may supply the destination (e.g. pinned
    memory)."""
    fill = cap if fill_tokens is None else int(fill_tokens)
    if out is None:
        out = torch.zeros((B, Hkv, cap, D), dtype=torch.bfloat16)
    jobs = []
    c = 0
    for b in range(B):
        for h in range(Hkv):
            for t0 in range(0, fill, chunk_tokens):
                t1 = min(fill, t0 + chunk_tokens)
                jobs.append((b, h, t0, t1, c))
                c += 1

    def run(job):
        b, h, t0, t1, cc = job
        out[b, h, t0:t1] = _cache_chunk(seed, cc, (t1 - t0) * D).view(t1 - t0, D)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(run, jobs))
    return out


def positions_uniform(B, lo, hi, seed=0):
    """int32 positions uniform in [lo, hi)."""
    g = _gen(seed)
    return torch.randint(int(lo), int(hi), (B,), generator=g, dtype=torch.int64).to(torch.int32)


WEIGHT_STD = 0.02   # projection weights ~ N(0, 0.02^2), a common initialiser scale
NORM_JITTER = 0.1   # RMSNorm weights ~ 1 + N(0, 0.1^2)


def block_weights(hidden, Hq, Hkv, D=256, seed=0):
    """Random weights of one attention block, CPU bf16: the RMSNorm weight
    [hidden], the fused q/k/v/g projection [(Hq + 2 Hkv) D + Hq, hidden] and
    out_proj [hidden, Hq D]. Draw order: norm, fused projection, out_proj."""
    g = _gen(seed)
    norm = (1.0 + NORM_JITTER * torch.randn(hidden, generator=g)).to(torch.bfloat16)
    qkvg = _normal(g, ((Hq + 2 * Hkv) * D + Hq, hidden), WEIGHT_STD)
    o = _normal(g, (hidden, Hq * D), WEIGHT_STD)
    return {"norm": norm, "qkvg": qkvg, "o": o}


def hidden_states(T, hidden, seed=0):
    """Block inputs x [T, hidden] ~ N(0, 1), fp32 (the residual stream)."""
    return torch.randn((T, hidden), generator=_gen(seed), dtype=torch.float32)
