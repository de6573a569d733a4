"""ctypes binding of libhattn.so (C ABI in include/hattn.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels. Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "hattn.h")

LAYER_SLIDING, LAYER_FULL = 0, 1
GATE_SIGMOID, GATE_SILU = 0, 1
KV_RING, KV_LINEAR, KV_PAGED = 0, 1, 2
HEAD_DIM = 256


class HattnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("layer_type", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("rotary_fraction", ctypes.c_double),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("gate_act", ctypes.c_int32),
    ]


class KvCacheC(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("kind", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
    ]


class BlockWeightsC(ctypes.Structure):
    _fields_ = [
        ("norm_weight", ctypes.c_void_p),
        ("qkvg_weight", ctypes.c_void_p),
        ("o_weight", ctypes.c_void_p),
        ("hidden", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
    ]


class KvLayerPlan(ctypes.Structure):
    _fields_ = [
        ("layer_type", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("k_offset", ctypes.c_uint64),
        ("v_offset", ctypes.c_uint64),
        ("bytes", ctypes.c_uint64),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "hattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "hattn_layer_defaults": (ctypes.c_int, [_I, _I, _I, ctypes.POINTER(LayerDesc)]),
    "hattn_rope_apply": (ctypes.c_int, [_P, _I, _I, _I, _P, ctypes.c_double, ctypes.c_double, _P]),
    "hattn_prefill_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.POINTER(KvCacheC), _I, _I]),
    "hattn_prefill": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _I, _I, _P,
                                     ctypes.POINTER(KvCacheC), _P, _P, ctypes.c_size_t, _P]),
    "hattn_prefill_varlen_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.POINTER(KvCacheC),
                                                              _I, _P]),
    "hattn_prefill_varlen": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _I, _P, _P,
                                            ctypes.POINTER(KvCacheC), _P, _P, ctypes.c_size_t, _P]),
    "hattn_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.POINTER(KvCacheC), _I]),
    "hattn_decode": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _I, _P, _I,
                                    ctypes.POINTER(KvCacheC), _P, _P, ctypes.c_size_t, _P]),
    "hattn_decode_static": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _I, _P, _I,
                                           ctypes.POINTER(KvCacheC), _P, _P]),
    "hattn_block_prefill_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.POINTER(BlockWeightsC),
                                                             ctypes.POINTER(KvCacheC), _I, _P]),
    "hattn_block_prefill": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(BlockWeightsC), _P, _I, _P, _P,
                                           ctypes.POINTER(KvCacheC), _P, _P, ctypes.c_size_t, _P]),
    "hattn_block_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc), ctypes.POINTER(BlockWeightsC),
                                                            ctypes.POINTER(KvCacheC), _I]),
    "hattn_block_decode": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(BlockWeightsC), _P, _I, _P, _I,
                                          ctypes.POINTER(KvCacheC), _P, _P, ctypes.c_size_t, _P]),
    "hattn_kv_plan": (ctypes.c_int, [_I, _P, _I, _I, _I, _I, ctypes.POINTER(KvLayerPlan),
                                     ctypes.POINTER(ctypes.c_uint64)]),
    "hattn_kv_cache_at": (ctypes.c_int, [ctypes.POINTER(KvLayerPlan), _P, ctypes.POINTER(KvCacheC)]),
    "hattn_debug_index_probe": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _I, _I, _I, _I, _P, _P, _P, _P]),
    "hattn_debug_read_probe": (ctypes.c_int, [_P, ctypes.c_size_t, _I, _P, _P]),
    "hattn_debug_mfma_probe": (ctypes.c_int, [_I, _I, _P, _P]),
    "hattn_debug_lds_probe": (ctypes.c_int, [_I, _I, _I, _P, _P]),
    "hattn_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "hattn_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]),
    "hattn_profile_read_clock": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double)]),
}
PROFILE_PREFILL, PROFILE_DECODE = 0, 1


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m full_gqa_attention_spark2_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/hattn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hattn_[a-z_0-9]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().hattn_status_string(status).decode()


def _check(fn, status):
    if status != 0:
        raise HattnError(fn, status, status_string(status))


def _stream(dev=None):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype=torch.bfloat16, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def layer_desc(layer_type, num_q_heads=16, num_kv_heads=4, **overrides) -> LayerDesc:
    """The page's parameters for a layer type ("sliding"/"full" or 0/1),
    with optional overrides of window / rope_theta / rotary_fraction /
    gate_act ("sigmoid"/"silu" or 0/1)."""
    lt = {"sliding": LAYER_SLIDING, "full": LAYER_FULL}.get(layer_type, layer_type)
    d = LayerDesc()
    _check("hattn_layer_defaults", lib().hattn_layer_defaults(lt, num_q_heads, num_kv_heads, ctypes.byref(d)))
    for k, v in overrides.items():
        if k == "gate_act":
            v = {"sigmoid": GATE_SIGMOID, "silu": GATE_SILU}.get(v, v)
        setattr(d, k, v)
    return d


class KVCache:
    """A layer's cache: K and V bf16 [B, Hkv, capacity, 256] on the GPU; or,
    for a paged cache (KVCache.paged), page pools [num_pages, Hkv,
    page_size, 256] with an int32 block table [B, capacity / page_size]."""

    def __init__(self, k, v, kind):
        self.k, self.v = k, v
        self.kind = {"ring": KV_RING, "linear": KV_LINEAR}.get(kind, kind)
        self.block_table = None
        _need(k, "cache.k")
        _need(v, "cache.v", shape=k.shape)
        if k.dim() != 4 or k.shape[3] != HEAD_DIM:
            raise ValueError("cache tensors must be [B, Hkv, capacity, 256]")
        self.batch, self.capacity = k.shape[0], k.shape[2]

    @classmethod
    def empty(cls, B, Hkv, capacity, kind, device="cuda"):
        k = torch.zeros((B, Hkv, capacity, HEAD_DIM), dtype=torch.bfloat16, device=device)
        return cls(k, torch.zeros_like(k), kind)

    @classmethod
    def paged(cls, k_pool, v_pool, block_table):
        """Pools bf16 [num_pages, Hkv, page_size, 256] and a device int32
        block table [B, pages_per_seq]: sequence b's slot p is row
        p % page_size of page block_table[b, p // page_size]."""
        c = cls.__new__(cls)
        _need(k_pool, "cache.k")
        _need(v_pool, "cache.v", shape=k_pool.shape)
        _need(block_table, "block_table", torch.int32)
        if k_pool.dim() != 4 or k_pool.shape[3] != HEAD_DIM or block_table.dim() != 2:
            raise ValueError("pools must be [num_pages, Hkv, page_size, 256], the table [B, pages]")
        c.k, c.v, c.kind, c.block_table = k_pool, v_pool, KV_PAGED, block_table
        c.page_size = k_pool.shape[2]
        c.batch, c.capacity = block_table.shape[0], block_table.shape[1] * c.page_size
        return c

    def c(self) -> KvCacheC:
        if self.kind == KV_PAGED:
            return KvCacheC(self.k.data_ptr(), self.v.data_ptr(), self.kind, self.batch, self.capacity,
                            self.page_size, self.block_table.data_ptr(), self.k.shape[0])
        return KvCacheC(self.k.data_ptr(), self.v.data_ptr(), self.kind, self.batch, self.capacity)


def prefill_workspace_size(desc, cache, B, S):
    cc = cache.c()
    return int(lib().hattn_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(cc), B, S))


def decode_workspace_size(desc, cache, B):
    cc = cache.c()
    return int(lib().hattn_decode_workspace_size(ctypes.byref(desc), ctypes.byref(cc), B))


def _workspace(nbytes, device, ws):
    if ws is not None:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def hattn_rope_apply(x, pos, theta, rotary_fraction):
    """In place RoPE of x bf16 [n_tok, n_heads, head_dim] at int32 pos [n_tok]."""
    _need(x, "x")
    _need(pos, "pos", torch.int32, (x.shape[0],))
    n_tok, n_heads, head_dim = x.shape
    _check("hattn_rope_apply", lib().hattn_rope_apply(_ptr(x), n_tok, n_heads, head_dim, _ptr(pos),
                                                       float(theta), float(rotary_fraction), _stream(x.device)))
    return x


def hattn_prefill(desc, q, k, v, gate, start_pos, cache, out=None, workspace=None):
    """Prefill of q [B,S,Hq,256], k/v [B,S,Hkv,256], gate [B,S,Hq] at host
    start positions; writes the new keys/values to ``cache``; returns out."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    _need(q, "q")
    _need(k, "k", shape=(B, S, Hkv, D))
    _need(v, "v", shape=(B, S, Hkv, D))
    _need(gate, "gate", shape=(B, S, Hq))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", shape=q.shape)
    sp = (ctypes.c_int32 * B)(*[int(x) for x in start_pos])
    cc = cache.c()
    ws = _workspace(prefill_workspace_size(desc, cache, B, S), q.device, workspace)
    _check("hattn_prefill", lib().hattn_prefill(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), B, S,
        ctypes.cast(sp, ctypes.c_void_p), ctypes.byref(cc), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(q.device)))
    return out


def hattn_prefill_varlen(desc, q, k, v, gate, cu_seqlens, start_pos, cache, out=None, workspace=None):
    """Ragged prefill over packed tokens: q [T,Hq,256], k/v [T,Hkv,256],
    gate [T,Hq]; host cu_seqlens [B+1] (sequence b = rows cu[b]..cu[b+1]-1)
    and start positions [B]; writes the new keys/values to ``cache``;
    returns out [T,Hq,256]."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    B = len(cu_seqlens) - 1
    _need(q, "q")
    _need(k, "k", shape=(T, Hkv, D))
    _need(v, "v", shape=(T, Hkv, D))
    _need(gate, "gate", shape=(T, Hq))
    if int(cu_seqlens[-1]) != T or len(start_pos) != B:
        raise ValueError("cu_seqlens[-1] must equal the packed token count and start_pos have B entries")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", shape=q.shape)
    cu = (ctypes.c_int32 * (B + 1))(*[int(x) for x in cu_seqlens])
    sp = (ctypes.c_int32 * B)(*[int(x) for x in start_pos])
    cc = cache.c()
    size = int(lib().hattn_prefill_varlen_workspace_size(ctypes.byref(desc), ctypes.byref(cc), B,
                                                         ctypes.cast(cu, ctypes.c_void_p)))
    ws = _workspace(size, q.device, workspace)
    _check("hattn_prefill_varlen", lib().hattn_prefill_varlen(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), B, ctypes.cast(cu, ctypes.c_void_p),
        ctypes.cast(sp, ctypes.c_void_p), ctypes.byref(cc), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(q.device)))
    return out


def hattn_decode(desc, q, k, v, gate, pos, max_pos, cache, out=None, workspace=None):
    """One decode step: q [B,Hq,256], k/v [B,Hkv,256], gate [B,Hq], device
    int32 positions pos [B] with host bound max_pos; returns out [B,Hq,256]."""
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(q, "q")
    _need(k, "k", shape=(B, Hkv, D))
    _need(v, "v", shape=(B, Hkv, D))
    _need(gate, "gate", shape=(B, Hq))
    _need(pos, "pos", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", shape=q.shape)
    cc = cache.c()
    ws = _workspace(decode_workspace_size(desc, cache, B), q.device, workspace)
    _check("hattn_decode", lib().hattn_decode(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), B, _ptr(pos), int(max_pos),
        ctypes.byref(cc), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device)))
    return out


DECODE_STATIC_SCRATCH_BYTES = 6 << 20   # HATTN_DECODE_STATIC_SCRATCH_BYTES


def hattn_decode_static(desc, q, k, v, gate, pos, max_pos, cache, out=None):
    """hattn_decode with the library's static scratch instead of a
    workspace (the call allocates nothing on the device; pass `out`)."""
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(q, "q")
    _need(k, "k", shape=(B, Hkv, D))
    _need(v, "v", shape=(B, Hkv, D))
    _need(gate, "gate", shape=(B, Hq))
    _need(pos, "pos", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", shape=q.shape)
    cc = cache.c()
    _check("hattn_decode_static", lib().hattn_decode_static(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), B, _ptr(pos), int(max_pos),
        ctypes.byref(cc), _ptr(out), _stream(q.device)))
    return out


class BlockWeights:
    """Weights of one attention block on the GPU (bf16): the input RMSNorm
    weight [hidden], the fused projection [(Hq + 2 Hkv) * 256 + Hq, hidden]
    (q_k_v_proj rows Q, K, V, then the g_proj rows) and out_proj [hidden,
    Hq * 256]."""

    def __init__(self, norm_weight, qkvg_weight, o_weight, rms_eps=1e-6):
        H = norm_weight.shape[0]
        _need(norm_weight, "norm_weight", shape=(H,))
        _need(qkvg_weight, "qkvg_weight")
        _need(o_weight, "o_weight")
        if qkvg_weight.dim() != 2 or qkvg_weight.shape[1] != H or o_weight.dim() != 2 or o_weight.shape[0] != H:
            raise ValueError("weight shapes do not match the hidden size")
        self.norm_weight, self.qkvg_weight, self.o_weight = norm_weight, qkvg_weight, o_weight
        self.hidden, self.rms_eps = H, float(rms_eps)

    def c(self) -> BlockWeightsC:
        return BlockWeightsC(self.norm_weight.data_ptr(), self.qkvg_weight.data_ptr(), self.o_weight.data_ptr(),
                             self.hidden, self.rms_eps)


def block_prefill_workspace_size(desc, weights, cache, cu_seqlens):
    B = len(cu_seqlens) - 1
    cu = (ctypes.c_int32 * (B + 1))(*[int(v) for v in cu_seqlens])
    cc, wc = cache.c(), weights.c()
    return int(lib().hattn_block_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(wc), ctypes.byref(cc), B,
                                                        ctypes.cast(cu, ctypes.c_void_p)))


def block_decode_workspace_size(desc, weights, cache, B):
    cc, wc = cache.c(), weights.c()
    return int(lib().hattn_block_decode_workspace_size(ctypes.byref(desc), ctypes.byref(wc), ctypes.byref(cc), B))


def hattn_block_prefill(desc, weights, x, cu_seqlens, start_pos, cache, out=None, workspace=None):
    """The attention block over packed new tokens x [T, hidden] (fp32, the
    residual stream; host cu_seqlens [B+1], start positions [B]); returns
    out [T, hidden] fp32 = x + out_proj(core(...)); out may be x."""
    T, H = x.shape
    B = len(cu_seqlens) - 1
    _need(x, "x", torch.float32, (T, weights.hidden))
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.float32, x.shape)
    cu = (ctypes.c_int32 * (B + 1))(*[int(v) for v in cu_seqlens])
    sp = (ctypes.c_int32 * B)(*[int(v) for v in start_pos])
    cc, wc = cache.c(), weights.c()
    ws = _workspace(block_prefill_workspace_size(desc, weights, cache, cu_seqlens), x.device, workspace)
    _check("hattn_block_prefill", lib().hattn_block_prefill(
        ctypes.byref(desc), ctypes.byref(wc), _ptr(x), B, ctypes.cast(cu, ctypes.c_void_p),
        ctypes.cast(sp, ctypes.c_void_p), ctypes.byref(cc), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(x.device)))
    return out


def hattn_block_decode(desc, weights, x, pos, max_pos, cache, out=None, workspace=None):
    """The attention block for one token per sequence, x [B, hidden] fp32,
    at device int32 positions pos [B]; returns out [B, hidden] fp32; out
    may be x."""
    B, H = x.shape
    _need(x, "x", torch.float32, (B, weights.hidden))
    _need(pos, "pos", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.float32, x.shape)
    cc, wc = cache.c(), weights.c()
    ws = _workspace(block_decode_workspace_size(desc, weights, cache, B), x.device, workspace)
    _check("hattn_block_decode", lib().hattn_block_decode(
        ctypes.byref(desc), ctypes.byref(wc), _ptr(x), B, _ptr(pos), int(max_pos), ctypes.byref(cc), _ptr(out),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(x.device)))
    return out


def hattn_kv_plan(n_layers, num_kv_heads, batch, max_tokens, window=512, layer_types=None):
    """Cache layout of a layer stack in one arena: (list of KvLayerPlan,
    arena bytes). layer_types: None (full iff i mod 4 == 3) or a sequence of
    "sliding"/"full" (or 0/1)."""
    plan = (KvLayerPlan * n_layers)()
    total = ctypes.c_uint64()
    lt = None
    if layer_types is not None:
        if len(layer_types) != n_layers:
            raise ValueError("layer_types must have n_layers entries")
        lt = (ctypes.c_int32 * n_layers)(*[{"sliding": LAYER_SLIDING, "full": LAYER_FULL}.get(t, t)
                                          for t in layer_types])
    _check("hattn_kv_plan", lib().hattn_kv_plan(n_layers, ctypes.cast(lt, ctypes.c_void_p) if lt else None,
                                                num_kv_heads, batch, max_tokens, window, plan,
                                                ctypes.byref(total)))
    return list(plan), int(total.value)


def kv_arena(arena_bytes, device="cuda"):
    """A device arena of the planned size (uint8, 256-byte aligned)."""
    return torch.empty(max(int(arena_bytes), 256), dtype=torch.uint8, device=device)


def kv_cache_at(layer_plan, arena):
    """The KVCache of one planned layer: K and V are bf16 views into the
    arena at the offsets hattn_kv_cache_at returns."""
    _need(arena, "arena", torch.uint8)
    cc = KvCacheC()
    _check("hattn_kv_cache_at", lib().hattn_kv_cache_at(ctypes.byref(layer_plan), _ptr(arena), ctypes.byref(cc)))
    shape = (cc.batch, layer_plan.num_kv_heads, cc.capacity, HEAD_DIM)
    n = cc.batch * layer_plan.num_kv_heads * cc.capacity * HEAD_DIM * 2
    base = arena.data_ptr()
    def view(ptr):
        off = ptr - base
        if off < 0 or off + n > arena.numel():
            raise ValueError("planned block lies outside the arena")
        return arena[off:off + n].view(torch.bfloat16).view(shape)
    return KVCache(view(cc.k), view(cc.v), cc.kind)


def hattn_debug_index_probe(desc, kind, capacity, q_pos0, n_q, device="cuda"):
    """Device-side mask [n_q, capacity] (uint8), key positions [n_q,
    capacity] (int32) and own-token slots [n_q] (int32) of a decode view."""
    kind = {"ring": KV_RING, "linear": KV_LINEAR}.get(kind, kind)
    mask = torch.empty((n_q, capacity), dtype=torch.uint8, device=device)
    key_pos = torch.empty((n_q, capacity), dtype=torch.int32, device=device)
    slot = torch.empty((n_q,), dtype=torch.int32, device=device)
    _check("hattn_debug_index_probe", lib().hattn_debug_index_probe(
        ctypes.byref(desc), kind, capacity, q_pos0, n_q, _ptr(mask), _ptr(key_pos), _ptr(slot),
        _stream(mask.device)))
    return mask, key_pos, slot


def hattn_profile_enable(enable=True):
    """Record HIP events around the attention kernels of later calls."""
    _check("hattn_profile_enable", lib().hattn_profile_enable(1 if enable else 0))


def hattn_profile_read(kind):
    """(count, total_ms) of the recorded kernel sections of one kind."""
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check("hattn_profile_read", lib().hattn_profile_read(kind, ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def hattn_profile_read_clock():
    """Average shader clock (GHz) of the prefill attention kernels profiled
    since the last read (0.0 when none were)."""
    g = ctypes.c_double()
    _check("hattn_profile_read_clock", lib().hattn_profile_read_clock(ctypes.byref(g)))
    return float(g.value)


def debug_read_probe(buf, blocks, sink):
    """Streams the bytes of device tensor buf with `blocks` blocks."""
    _check("hattn_debug_read_probe", lib().hattn_debug_read_probe(
        _ptr(buf), buf.numel() * buf.element_size(), blocks, _ptr(sink), _stream(buf.device)))


def debug_mfma_probe(blocks, iters, sink):
    """Back-to-back bf16 MFMA 32x32x16 in `blocks` four-wave blocks."""
    _check("hattn_debug_mfma_probe", lib().hattn_debug_mfma_probe(blocks, iters, _ptr(sink), _stream(sink.device)))


def debug_lds_probe(mode, blocks, iters, out):
    """LDS fragment reads (mode 0 b128, 1 transposed b64, 2 mixed with MFMA) in
    `blocks` four-wave blocks; out: int64 device tensor [blocks][2], [b][0] =
    elapsed shader clock ticks of block b."""
    _check("hattn_debug_lds_probe", lib().hattn_debug_lds_probe(mode, blocks, iters, _ptr(out), _stream(out.device)))
