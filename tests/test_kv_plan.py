"""The KV planner (hattn_kv_plan / hattn_kv_cache_at): pure host arithmetic,
checked against the page's KV-cache table (tests/golden/kv_cache_sizing.json,
page "Spark-X2.5 架构（4B / 1.7B）" §6) and the oracle's sizing and layer
schedule. No device memory is touched.
"""
import ctypes
import json
import os

import pytest

from full_gqa_attention_spark2_amd import binding as hb
from oracle import hattn_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ARENA = 0x100000  # 256-byte aligned address, never dereferenced


def _golden():
    with open(os.path.join(GOLDEN, "kv_cache_sizing.json")) as f:
        return json.load(f)


def _check_layout(plan, arena_bytes):
    prev_end = 0
    for e in plan:
        blk = e.batch * e.num_kv_heads * e.capacity * 256 * 2
        assert e.bytes == 2 * blk
        assert e.k_offset % 256 == 0 and e.v_offset % 256 == 0
        assert e.k_offset >= prev_end and e.v_offset >= e.k_offset + blk
        prev_end = e.v_offset + blk
    assert prev_end <= arena_bytes < prev_end + 256


def test_plan_matches_page_table_4b_and_1p7b():
    t = _golden()
    T = t["tokens"]
    plan, total = hb.hattn_kv_plan(36, 4, 1, T)
    _check_layout(plan, total)
    assert [("full" if e.layer_type == hb.LAYER_FULL else "sliding") for e in plan] == O.layer_schedule(36)
    full = sum(e.bytes for e in plan if e.layer_type == hb.LAYER_FULL)
    sliding = sum(e.bytes for e in plan if e.layer_type == hb.LAYER_SLIDING)
    rows = {r["what"]: r for r in t["rows"]}
    for what, got in (("9 full layers at 1M tokens (4B)", full), ("27 sliding layers capped at 512 (4B)", sliding)):
        r = rows[what]
        assert abs(got / r["page_value_bytes"] - 1) <= r["rel_tol"], what
    assert total == O.kv_bytes_model(36, 4, T)       # every block is a multiple of 256 bytes
    for e in plan:
        kept = T if e.layer_type == hb.LAYER_FULL else 512
        assert e.bytes == kept * t["bytes_per_token_per_layer_4B"]
        assert (e.kind, e.capacity) == ((hb.KV_LINEAR, T) if e.layer_type == hb.LAYER_FULL else (hb.KV_RING, 512))
    # all layers full: the page's 147 GB, and the hybrid stack is ~1/4 of it
    allf, total_f = hb.hattn_kv_plan(36, 4, 1, T, layer_types=["full"] * 36)
    r = rows["all 36 layers full at 1M tokens (4B)"]
    assert abs(total_f / r["page_value_bytes"] - 1) <= r["rel_tol"]
    assert abs(total / total_f - t["ratio_hybrid_over_all_full"]) <= t["ratio_rel_tol"]
    # 1.7B: 28 layers, 2 KV heads, 7 full layers
    plan, total = hb.hattn_kv_plan(28, 2, 1, T)
    full = sum(e.bytes for e in plan if e.layer_type == hb.LAYER_FULL)
    r = rows["7 full layers at 1M tokens (1.7B)"]
    assert abs(full / r["page_value_bytes"] - 1) <= r["rel_tol"]
    assert total == O.kv_bytes_model(28, 2, T)
    # the explainer page's 144 GiB: all 36 layers full at 2^20 tokens
    _, total_f = hb.hattn_kv_plan(36, 4, 1, 1 << 20, layer_types=[1] * 36)
    assert total_f == t["all_full_2pow20_GiB_explainer_page"] * 2 ** 30


def test_plan_short_context_batch_and_custom_types():
    # max_tokens <= window: sliding layers need no ring, a linear cache of max_tokens
    plan, total = hb.hattn_kv_plan(8, 4, 3, 300)
    _check_layout(plan, total)
    assert all(e.kind == hb.KV_LINEAR and e.capacity == 300 and e.batch == 3 for e in plan)
    plan, total = hb.hattn_kv_plan(8, 4, 3, 513)
    assert [e.kind for e in plan] == [hb.KV_RING] * 3 + [hb.KV_LINEAR] + [hb.KV_RING] * 3 + [hb.KV_LINEAR]
    # a custom schedule and window; odd sizes get padded to 256-byte blocks
    plan, total = hb.hattn_kv_plan(3, 1, 1, 1001, window=7, layer_types=["full", "sliding", "full"])
    _check_layout(plan, total)
    assert [(e.kind, e.capacity) for e in plan] == [(hb.KV_LINEAR, 1001), (hb.KV_RING, 7), (hb.KV_LINEAR, 1001)]
    assert total == sum(-(-e.bytes // 2 // 256) * 256 * 2 for e in plan)


def test_plan_rejects_bad_arguments():
    L = hb.lib()
    plan = (hb.KvLayerPlan * 4)()
    total = ctypes.c_uint64()
    bad_types = (ctypes.c_int32 * 4)(0, 1, 2, 0)
    f = L.hattn_kv_plan
    assert f(4, None, 4, 1, 100, 512, None, ctypes.byref(total)) == -1
    assert f(4, None, 4, 1, 100, 512, plan, None) == -1
    assert f(0, None, 4, 1, 100, 512, plan, ctypes.byref(total)) == -2
    assert f(4, None, 0, 1, 100, 512, plan, ctypes.byref(total)) == -2
    assert f(4, None, 4, 0, 100, 512, plan, ctypes.byref(total)) == -2
    assert f(4, None, 4, 1, 0, 512, plan, ctypes.byref(total)) == -2
    assert f(4, None, 4, 1, (1 << 30) + 1, 512, plan, ctypes.byref(total)) == -2
    assert f(4, None, 4, 1, 100, 0, plan, ctypes.byref(total)) == -5
    assert f(4, ctypes.cast(bad_types, ctypes.c_void_p), 4, 1, 100, 512, plan, ctypes.byref(total)) == -2


def test_cache_at_points_into_the_arena():
    L = hb.lib()
    plan, total = hb.hattn_kv_plan(4, 4, 2, 2000)
    for e in plan:
        c = hb.KvCacheC()
        assert L.hattn_kv_cache_at(ctypes.byref(e), ARENA, ctypes.byref(c)) == 0
        assert (c.k, c.v) == (ARENA + e.k_offset, ARENA + e.v_offset)
        assert (c.kind, c.batch, c.capacity) == (e.kind, 2, e.capacity)
        # the cache passes the layer's own validation (a workspace size, no launch)
        desc = hb.layer_desc("full" if e.layer_type == hb.LAYER_FULL else "sliding")
        assert L.hattn_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(c), 2, 100) > 0
    c = hb.KvCacheC()
    assert L.hattn_kv_cache_at(ctypes.byref(plan[0]), ARENA + 16, ctypes.byref(c)) == -9
    assert L.hattn_kv_cache_at(ctypes.byref(plan[0]), None, ctypes.byref(c)) == -1
    e = hb.KvLayerPlan.from_buffer_copy(plan[1])
    e.v_offset = e.k_offset + 256          # V overlapping K
    assert L.hattn_kv_cache_at(ctypes.byref(e), ARENA, ctypes.byref(c)) == -2
    e = hb.KvLayerPlan.from_buffer_copy(plan[1])
    e.bytes += 2
    assert L.hattn_kv_cache_at(ctypes.byref(e), ARENA, ctypes.byref(c)) == -2
