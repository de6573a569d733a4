"""Host-side checks of the C ABI: the library loads, exports every function
the header declares, and rejects bad arguments with the documented status
before touching the device. No kernel is launched here.
"""
import ctypes
import json
import os

import pytest
import torch

from full_gqa_attention_spark2_amd import binding as hb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# Most calls below are built to fail validation; on a machine with a GPU the
# fake pointers would be dangerous if a check were missing, so those tests
# only run where no GPU is visible. The export, status-string and
# layer-default checks launch nothing and run everywhere.
fake_pointers = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only ABI checks use fake pointers")

FAKE = 0x10000  # aligned, never dereferenced


@pytest.fixture(scope="module")
def L():
    return hb.lib()


def test_exports_every_header_function(L):
    names = hb.header_functions()
    assert {"hattn_rope_apply", "hattn_prefill", "hattn_decode"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(0, -12, -1):
        s = hb.status_string(code)
        assert s and s != "unknown status"
    assert hb.status_string(-99) == "unknown status"


def test_layer_defaults_match_page_tables():
    with open(os.path.join(GOLDEN, "spark_layer_config.json")) as f:
        t = json.load(f)
    s = hb.layer_desc("sliding", 16, 4)
    assert (s.window, s.rope_theta, s.rotary_fraction) == (
        t["models"]["4B"]["sliding_window"], t["rope"]["sliding"]["rope_theta"], t["rope"]["sliding"]["partial_rotary_factor"])
    f_ = hb.layer_desc("full", 8, 2)
    assert f_.window <= 0
    assert (f_.rope_theta, f_.rotary_fraction, f_.head_dim) == (
        t["rope"]["full"]["rope_theta"], t["rope"]["full"]["partial_rotary_factor"], 256)
    assert s.gate_act == f_.gate_act == hb.GATE_SIGMOID       # Eq. 1 and both checkpoints
    assert hb.layer_desc("full", gate_act="silu").gate_act == hb.GATE_SILU
    assert ctypes.sizeof(hb.LayerDesc) == 40                  # the C struct's size


def _prefill(L, desc, cache, B=1, S=8, start=(0,), ws_bytes=1 << 30, q=FAKE, ws=FAKE, gate=FAKE):
    sp = (ctypes.c_int32 * len(start))(*start)
    return L.hattn_prefill(ctypes.byref(desc), q, FAKE, FAKE, gate, B, S, ctypes.cast(sp, ctypes.c_void_p),
                           ctypes.byref(cache) if cache is not None else None, FAKE, ws, ws_bytes, None)


def _decode(L, desc, cache, B=1, max_pos=10, ws_bytes=1 << 30, pos=FAKE):
    return L.hattn_decode(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, B, pos, max_pos,
                          ctypes.byref(cache), FAKE, FAKE, ws_bytes, None)


@fake_pointers
def test_prefill_rejects_bad_arguments(L):
    sl = hb.layer_desc("sliding")
    fu = hb.layer_desc("full")
    ring = hb.KvCacheC(FAKE, FAKE, hb.KV_RING, 1, 512)
    lin = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 64)
    E = hb
    cases = []
    d = hb.layer_desc("sliding"); d.head_dim = 128; cases.append((d, ring, {}, -3))
    d = hb.layer_desc("sliding"); d.num_q_heads = 8; cases.append((d, ring, {}, -3))      # group 2
    d = hb.layer_desc("sliding"); d.num_q_heads = 15; cases.append((d, ring, {}, -2))     # not a multiple
    d = hb.layer_desc("sliding"); d.rotary_fraction = 0.3; cases.append((d, ring, {}, -4))
    d = hb.layer_desc("sliding"); d.rope_theta = -1.0; cases.append((d, ring, {}, -4))
    d = hb.layer_desc("sliding"); d.window = 0; cases.append((d, ring, {}, -5))
    d = hb.layer_desc("full"); d.window = 512; cases.append((d, lin, {}, -5))
    d = hb.layer_desc("full"); d.gate_act = 2; cases.append((d, lin, {}, -3))            # unknown gate mode
    d = hb.layer_desc("full"); d.gate_act = -1; cases.append((d, lin, {}, -3))
    cases.append((fu, ring, {}, -6))                                                   # ring on a full layer
    cases.append((sl, hb.KvCacheC(FAKE, FAKE, hb.KV_RING, 1, 256), {}, -6))              # ring cap != window
    cases.append((sl, hb.KvCacheC(FAKE, FAKE, hb.KV_RING, 2, 512), {}, -6))              # batch mismatch
    cases.append((sl, hb.KvCacheC(FAKE, FAKE, 7, 1, 512), {}, -6))                       # unknown kind
    cases.append((fu, lin, {"start": (60,)}, -7))                                      # 60 + 8 > 64
    cases.append((fu, lin, {"start": (-1,)}, -11))
    cases.append((fu, lin, {"ws_bytes": 16}, -8))
    cases.append((fu, lin, {"ws": 0}, -8))
    cases.append((fu, lin, {"q": FAKE + 2}, -9))
    cases.append((fu, lin, {"q": 0}, -1))
    cases.append((fu, hb.KvCacheC(0, FAKE, hb.KV_LINEAR, 1, 64), {}, -1))
    cases.append((fu, lin, {"B": 0, "start": (0,)}, -2))
    cases.append((fu, hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 200, 64), {"B": 200, "start": (0,) * 200}, -3))
    big = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, (1 << 23) + 1)
    cases.append((fu, big, {}, -3))                                                    # 32-bit row offsets
    cases.append((sl, ring, {"S": (1 << 23) - 510}, -3))                                 # 511 + S rows
    d = hb.layer_desc("full"); d.num_q_heads = 65540; d.num_kv_heads = 16385
    cases.append((d, lin, {}, -3))                                                     # 32-bit query row offsets
    for desc, cache, kw, want in cases:
        got = _prefill(L, desc, cache, **kw)
        assert got == want, (desc.layer_type, kw, got, want)


def _varlen(L, desc, cache, cu, start, ws_bytes=1 << 30):
    B = len(cu) - 1
    cu_a = (ctypes.c_int32 * len(cu))(*cu)
    sp = (ctypes.c_int32 * B)(*start)
    return L.hattn_prefill_varlen(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, B, ctypes.cast(cu_a, ctypes.c_void_p),
                                  ctypes.cast(sp, ctypes.c_void_p), ctypes.byref(cache), FAKE, FAKE, ws_bytes,
                                  None)


@fake_pointers
def test_paged_cache_validation(L):
    assert ctypes.sizeof(hb.KvCacheC) == 48
    fu = hb.layer_desc("full")
    sl = hb.layer_desc("sliding")
    def paged(cap=4096, ps=256, table=FAKE, pages=64, B=1):
        return hb.KvCacheC(FAKE, FAKE, hb.KV_PAGED, B, cap, ps, table, pages)
    # prefill: sliding layers take no paged cache; page size a multiple of 64
    # dividing the capacity; at most 4096 pages per sequence; a table
    assert _prefill(L, sl, paged()) == -6
    assert _prefill(L, fu, paged(ps=96, cap=96 * 40)) == -6
    assert _prefill(L, fu, paged(ps=256, cap=4096 + 64)) == -6
    assert _prefill(L, fu, paged(ps=64, cap=64 * 4097)) == -6
    assert _prefill(L, fu, paged(pages=0)) == -6
    assert _prefill(L, fu, paged(table=0)) == -1
    assert _prefill(L, fu, paged(table=FAKE + 2)) == -9
    assert _prefill(L, fu, paged(), start=(4090,)) == -7          # 4090 + 8 > 4096
    assert _decode(L, fu, paged(), max_pos=4096) == -7
    assert _decode(L, fu, paged(ps=32, cap=320)) == -6
    # workspace: the cos/sin table only (no staging)
    assert L.hattn_prefill_workspace_size(ctypes.byref(fu), ctypes.byref(paged()), 1, 100) == 100 * 32 * 8


@fake_pointers
def test_prefill_varlen_rejects_bad_arguments(L):
    fu = hb.layer_desc("full")
    lin = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 3, 64)
    assert _varlen(L, fu, lin, [1, 5, 9, 12], [0, 0, 0]) == -2          # not zero-based
    assert _varlen(L, fu, lin, [0, 5, 4, 12], [0, 0, 0]) == -2          # decreasing
    assert _varlen(L, fu, lin, [0, 5, 9, 12], [0, 61, 0]) == -7         # 61 + 4 > 64
    assert _varlen(L, fu, lin, [0, 5, 9, 12], [0, -1, 0]) == -11
    assert _varlen(L, fu, lin, [0, 5, 9, 12], [0, 0, 0], ws_bytes=16) == -8
    assert _varlen(L, fu, hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 2, 64), [0, 5, 9, 12], [0, 0, 0]) == -6
    assert _varlen(L, fu, lin, [0, 0, 0, 0], [0, 0, 0]) == 0            # nothing to do
    sp = (ctypes.c_int32 * 3)(0, 0, 0)
    assert L.hattn_prefill_varlen(ctypes.byref(fu), FAKE, FAKE, FAKE, FAKE, 3, None, ctypes.cast(sp, ctypes.c_void_p),
                                  ctypes.byref(lin), FAKE, FAKE, 1 << 30, None) == -1
    # workspace: the cos/sin table of the packed tokens (r/2 fp32 pairs each);
    # a ring adds K/V staging of window - 1 + the longest sequence's rows
    cu = (ctypes.c_int32 * 4)(0, 100, 130, 400)
    assert L.hattn_prefill_varlen_workspace_size(ctypes.byref(fu), ctypes.byref(lin), 3,
                                                 ctypes.cast(cu, ctypes.c_void_p)) == 400 * 32 * 8
    sl = hb.layer_desc("sliding")
    ring = hb.KvCacheC(FAKE, FAKE, hb.KV_RING, 3, 512)
    got = L.hattn_prefill_varlen_workspace_size(ctypes.byref(sl), ctypes.byref(ring), 3, ctypes.cast(cu, ctypes.c_void_p))
    assert got == 400 * 128 * 8 + 2 * 3 * 4 * (511 + 270) * 256 * 2


@fake_pointers
def test_block_rejects_bad_arguments(L):
    fu = hb.layer_desc("full")
    lin = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 2, 4096)
    cu = (ctypes.c_int32 * 3)(0, 100, 130)
    sp = (ctypes.c_int32 * 2)(0, 0)
    def pre(w, x=FAKE, out=FAKE, ws_bytes=1 << 34):
        return L.hattn_block_prefill(ctypes.byref(fu), ctypes.byref(w) if w is not None else None, x, 2,
                                     ctypes.cast(cu, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                                     ctypes.byref(lin), out, FAKE, ws_bytes, None)
    good = hb.BlockWeightsC(FAKE, FAKE, FAKE, 2560, 1e-6)
    assert pre(None) == -1
    assert pre(hb.BlockWeightsC(0, FAKE, FAKE, 2560, 1e-6)) == -1
    assert pre(hb.BlockWeightsC(FAKE, FAKE, FAKE, 2561, 1e-6)) == -2      # hidden not a multiple of 8
    assert pre(hb.BlockWeightsC(FAKE, FAKE, FAKE, 2560, 0.0)) == -2       # eps must be positive
    assert pre(hb.BlockWeightsC(FAKE, FAKE + 8, FAKE, 2560, 1e-6)) == -9
    assert pre(good, x=0) == -1
    assert pre(good, x=FAKE + 2) == -9
    assert pre(good, ws_bytes=1024) == -8
    # workspace: h, the fused projection, the core's output, out_proj's
    # output, 32 MiB of GEMM workspace, then the core's own (cos/sin table)
    T, H, n1 = 130, 2560, (16 + 8) * 256 + 16
    a = lambda b: (b + 255) // 256 * 256
    want = a(T * H * 2) + a(T * n1 * 2) + a(T * 4096 * 2) + a(T * H * 2) + (32 << 20) + a(T * 32 * 8)
    got = L.hattn_block_prefill_workspace_size(ctypes.byref(fu), ctypes.byref(good), ctypes.byref(lin), 2,
                                               ctypes.cast(cu, ctypes.c_void_p))
    assert got == want
    dec = L.hattn_block_decode(ctypes.byref(fu), ctypes.byref(hb.BlockWeightsC(FAKE, FAKE, FAKE, 0, 1e-6)), FAKE, 2,
                               FAKE, 10, ctypes.byref(lin), FAKE, FAKE, 1 << 34, None)
    assert dec == -2

    # the layer descriptor and the cache are validated before any workspace
    # arithmetic or launch, in both block entry points
    def pre_with(desc, cache):
        return L.hattn_block_prefill(ctypes.byref(desc), ctypes.byref(good), FAKE, 2, ctypes.cast(cu, ctypes.c_void_p),
                                     ctypes.cast(sp, ctypes.c_void_p), ctypes.byref(cache), FAKE, FAKE, 1 << 34, None)

    def dec_with(desc, cache):
        return L.hattn_block_decode(ctypes.byref(desc), ctypes.byref(good), FAKE, 2, FAKE, 10, ctypes.byref(cache),
                                    FAKE, FAKE, 1 << 34, None)

    sl = hb.layer_desc("sliding")
    g2 = hb.layer_desc("full", 8, 2)
    g2.num_kv_heads = 4                                                       # GQA group 2
    bad = [
        (g2, lin, -3),
        (fu, hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 4096), -6),           # cache batch 1 for B = 2
        (sl, hb.KvCacheC(FAKE, FAKE, hb.KV_RING, 2, 100), -6),              # ring capacity != window
        (fu, hb.KvCacheC(0, FAKE, hb.KV_LINEAR, 2, 4096), -1),              # null k
        (fu, hb.KvCacheC(FAKE, FAKE, hb.KV_PAGED, 2, 4096, 256, 0, 64), -1),  # paged, null block table
    ]
    for desc, cache, want in bad:
        assert pre_with(desc, cache) == want, (desc.num_kv_heads, cache.kind, cache.batch)
        assert dec_with(desc, cache) == want, (desc.num_kv_heads, cache.kind, cache.batch)
    assert L.hattn_block_prefill_workspace_size(ctypes.byref(g2), ctypes.byref(good), ctypes.byref(lin), 2,
                                                ctypes.cast(cu, ctypes.c_void_p)) == 0
    assert L.hattn_block_decode_workspace_size(ctypes.byref(fu), ctypes.byref(good),
                                               ctypes.byref(hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 4096)), 2) == 0


@fake_pointers
def test_decode_rejects_bad_arguments(L):
    sl = hb.layer_desc("sliding")
    fu = hb.layer_desc("full")
    lin = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 64)
    assert _decode(L, fu, lin, max_pos=64) == -7       # beyond capacity
    assert _decode(L, fu, lin, max_pos=-1) == -11
    assert _decode(L, fu, lin, pos=FAKE + 2) == -9
    assert _decode(L, fu, lin, pos=0) == -1
    assert _decode(L, sl, hb.KvCacheC(FAKE, FAKE, hb.KV_RING, 1, 100)) == -6
    assert _decode(L, hb.layer_desc("full", gate_act=3), lin) == -3
    big = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 1 << 20)
    assert _decode(L, fu, big, max_pos=(1 << 20) - 1, ws_bytes=100) == -8


@fake_pointers
def test_rope_apply_rejects_bad_arguments(L):
    f = L.hattn_rope_apply
    assert f(FAKE, 4, 2, 256, FAKE, 1e4, 0.3, None) == -4
    assert f(FAKE, 4, 2, 256, FAKE, 0.0, 1.0, None) == -4
    assert f(FAKE, 4, 2, 1024, FAKE, 1e4, 1.0, None) == -3
    assert f(FAKE, 4, 2, 255, FAKE, 1e4, 1.0, None) == -2
    assert f(0, 4, 2, 256, FAKE, 1e4, 1.0, None) == -1
    assert f(FAKE + 1, 4, 2, 256, FAKE, 1e4, 1.0, None) == -9
    assert f(0, 0, 2, 256, 0, 1e4, 1.0, None) == 0      # nothing to do


@fake_pointers
def test_workspace_sizes(L):
    fu = hb.layer_desc("full")
    sl = hb.layer_desc("sliding")
    lin = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 8192)
    ring = hb.KvCacheC(FAKE, FAKE, hb.KV_RING, 1, 512)
    # linear prefill: only the cos/sin table of the new positions (r/2 pairs of fp32)
    assert L.hattn_prefill_workspace_size(ctypes.byref(fu), ctypes.byref(lin), 1, 8192) == 8192 * 32 * 8
    # ring prefill: the table plus K/V staging of (window - 1 + S) rows
    got = L.hattn_prefill_workspace_size(ctypes.byref(sl), ctypes.byref(ring), 1, 1024)
    assert got == 1024 * 128 * 8 + 2 * 4 * (511 + 1024) * 256 * 2
    # decode over a 2^20-token linear cache needs split partials
    big = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 1 << 20)
    assert L.hattn_decode_workspace_size(ctypes.byref(fu), ctypes.byref(big), 1) >= 16 * 2 * 256 * 4
    assert L.hattn_prefill_workspace_size(None, ctypes.byref(lin), 1, 8) == 0


@fake_pointers
@pytest.mark.parametrize("layer,kind,cap,B,Hq,Hkv", [
    ("full", hb.KV_LINEAR, 266240, 2, 8, 2),     # the 1.7B full layer's 4096 + 262144 slots
    ("full", hb.KV_LINEAR, 4100, 8, 16, 4),
    ("full", hb.KV_LINEAR, 1 << 20, 1, 16, 4),
    ("sliding", hb.KV_LINEAR, 300000, 50, 16, 4),
    ("sliding", hb.KV_RING, 512, 3, 16, 4),
])
def test_decode_workspace_size_covers_every_position(L, layer, kind, cap, B, Hq, Hkv):
    """The size query is an upper bound: a decode at any max_pos the cache
    holds passes the workspace check with exactly that many bytes (here it
    then reaches the launch, which fails without a GPU)."""
    d = hb.layer_desc(layer, Hq, Hkv)
    if layer == "sliding" and kind == hb.KV_LINEAR:
        d.window = 1000
    c = hb.KvCacheC(FAKE, FAKE, kind, B, cap)
    ws = L.hattn_decode_workspace_size(ctypes.byref(d), ctypes.byref(c), B)
    assert ws > 0
    top = cap - 1 if kind != hb.KV_RING else (1 << 30) - 1
    probes = sorted(set([0, 1, 127, 128, 129, 1000, 4095, 131071, 262143, 262144, top] +
                        [int(x) for x in __import__("numpy").linspace(0, min(top, cap - 1 if kind != hb.KV_RING else 5000), 200)]))
    for mp in probes:
        if mp > top:
            continue
        st = _decode(L, d, c, B=B, max_pos=mp, ws_bytes=ws)
        assert st in (0, -10), (mp, st)


@fake_pointers
def test_decode_static_validates_before_using_its_scratch(L):
    """hattn_decode_static checks its arguments like hattn_decode before it
    looks up the static array (here the valid call then fails at the launch,
    without a GPU)."""
    fu = hb.layer_desc("full")
    def st(desc, cache, B=1, max_pos=10, pos=FAKE):
        return L.hattn_decode_static(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, B, pos, max_pos,
                                     ctypes.byref(cache), FAKE, None)
    lin = hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 1, 1 << 20)
    g2 = hb.layer_desc("full", 8, 2)
    g2.num_kv_heads = 4
    assert st(g2, lin) == -3
    assert st(fu, hb.KvCacheC(FAKE, FAKE, hb.KV_LINEAR, 2, 4096)) == -6
    assert st(fu, lin, max_pos=1 << 20) == -7
    assert st(fu, lin, pos=0) == -1
    assert st(fu, lin, max_pos=(1 << 20) - 1) == -10      # valid: reaches the launch


@fake_pointers
def test_measurement_probes_reject_bad_arguments(L):
    # modes, counts and the output pointer are checked before any launch
    lds = L.hattn_debug_lds_probe
    assert lds(3, 1, 1, FAKE, None) == -2
    assert lds(-1, 1, 1, FAKE, None) == -2
    assert lds(0, 0, 1, FAKE, None) == -2
    assert lds(0, 1, 0, FAKE, None) == -2
    assert lds(0, 1, 1, None, None) == -1
    assert lds(0, 1, 1, FAKE + 4, None) == -9
    assert L.hattn_debug_mfma_probe(0, 1, FAKE, None) == -2
    assert L.hattn_debug_mfma_probe(1, 1, None, None) == -1
    assert L.hattn_debug_read_probe(FAKE, 24, 1, FAKE, None) == -2
