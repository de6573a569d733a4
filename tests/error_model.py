"""A CPU model of where a bf16-MFMA attention pipeline rounds, used to size
the error budget against the fp64 oracle (test-side design tool; not the
oracle and not the GPU path).

The model follows the pages' definition (page "Spark-X2.5 架构（4B / 1.7B）",
§3 Eq. 1; §4 RoPE) in fp64 and inserts only the roundings such a pipeline
makes:
  - the rotated queries enter the score product as bf16 (or as a bf16 high
    part plus a bf16 low part, q_split=True);
  - the probabilities enter the P.V product as bf16 relative to the row max
    (or split into high and low parts, p_split=True); the softmax sum uses
    them unrounded;
  - the gated output is stored as bf16 (round to nearest even).
Keys are the cached bf16 keys in both the model and the oracle. fp32
accumulation is not modelled (its error is orders of magnitude smaller).
"""
import numpy as np

from oracle import hattn_oracle as O


def _split(x, split):
    hi = O.bf16_rne(x)
    return hi + O.bf16_rne(x - hi) if split else hi


def prefill_rows(q, k, v, gate, start, *, window, theta, rotary_fraction, rows, hist_k=None, hist_v=None,
                 hist_pos=None, q_split=False, p_split=False, q_scale=1.0):
    """Modelled outputs [len(rows), Hq, D] of one sequence (b = 0) of a
    prefill, in fp64 after the final bf16 rounding."""
    q = O.f64(q)[0] * q_scale
    k = O.f64(k)[0]
    v = O.f64(v)[0]
    g = O.f64(gate)[0]
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    pos = start + np.arange(S, dtype=np.int64)
    q_rot = _split(O.rope(q, pos, theta, rotary_fraction)[rows], q_split)
    k_hat = O.bf16_rne(O.rope(k, pos, theta, rotary_fraction))
    key_pos = pos if hist_k is None else np.concatenate([np.asarray(hist_pos, np.int64), pos])
    ok = O.allowed(pos[rows][:, None], key_pos[None, :], window)
    out = np.zeros((len(rows), Hq, D))
    for kv in range(Hkv):
        keys, vals = k_hat[:, kv], v[:, kv]
        if hist_k is not None:
            keys = np.concatenate([O.f64(hist_k[kv]), keys])
            vals = np.concatenate([O.f64(hist_v[kv]), vals])
        for h in range(kv * G, (kv + 1) * G):
            s = np.where(ok, (q_rot[:, h] @ keys.T) / 16.0, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o = (_split(p, p_split) @ vals) / p.sum(axis=1, keepdims=True)
            out[:, h] = O.bf16_rne(o * O.gate_factor(g[rows, h])[:, None])
    return out


def rel_rms(a, ref):
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def beyond_store(a, ref):
    """Max-abs error beyond what the bf16 store alone may add at |ref| >= 2
    (half a bf16 ulp of |ref| minus 2^-8; the GPU parity tests widen each
    element's bar by this outside the headline workloads)."""
    r = np.abs(ref)
    e = np.floor(np.log2(np.maximum(r, 2.0 ** -126)))
    return float((np.abs(a - ref) - np.maximum(0.0, 2.0 ** (e - 8) - 2.0 ** -8)).max())
