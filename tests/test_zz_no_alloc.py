"""hattn_decode_static (decode with the library's static scratch, no caller
workspace) against hattn_decode with a caller workspace, through the C ABI.

Two calls in a row on one GPU, the second smaller than the first, so the
second runs over the partials the first left in the shared array. Both entry
points run the same kernels and plan, so output rows and cache writes must be
bit-identical (stricter than the oracle tolerance that hattn_decode itself is
held to elsewhere).
"""
import numpy as np
import pytest
import torch

from full_gqa_attention_spark2_amd import binding as hb
from full_gqa_attention_spark2_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(layer, B, cap, kind, pos, seed):
    Hq, Hkv = 16, 4
    desc = hb.layer_desc(layer, Hq, Hkv)
    inp = {k: v.to(DEV) for k, v in synth.decode_inputs(B, Hq, Hkv, seed=seed).items()}
    ck = synth.cache_tensor(B, Hkv, cap, seed=seed + 1, threads=16).to(DEV)
    cv = synth.cache_tensor(B, Hkv, cap, seed=seed + 2, threads=16).to(DEV)
    pos_d = torch.as_tensor(pos, dtype=torch.int32).to(DEV)
    return desc, inp, ck, cv, pos_d, int(max(pos))


def _run_both(desc, inp, ck, cv, pos_d, max_pos, kind):
    c_ws = hb.KVCache(ck.clone(), cv.clone(), kind)
    c_st = hb.KVCache(ck.clone(), cv.clone(), kind)
    out_ws = hb.hattn_decode(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos_d, max_pos, c_ws)
    out_st = torch.full_like(inp["q"], float("nan"))
    hb.hattn_decode_static(desc, inp["q"], inp["k"], inp["v"], inp["gate"], pos_d, max_pos, c_st, out=out_st)
    torch.cuda.synchronize()
    return out_ws, out_st, c_ws, c_st


def _check(tag, out_ws, out_st, c_ws, c_st):
    a = out_ws.view(torch.int16).cpu().numpy()
    b = out_st.view(torch.int16).cpu().numpy()
    diff = int(np.count_nonzero(a != b))
    finite = bool(torch.isfinite(out_st.float()).all())
    print(f"{tag}: differing output values {diff} of {a.size}, all finite {finite}", flush=True)
    assert finite
    assert diff == 0
    assert torch.equal(c_ws.k.view(torch.int16), c_st.k.view(torch.int16))
    assert torch.equal(c_ws.v.view(torch.int16), c_st.v.view(torch.int16))


def test_static_scratch_decode_matches_workspace_decode_twice():
    # 1: full layer, B = 2 over 131072-slot linear caches (128 splits:
    #    4 MiB of partials in the static array)
    pos1 = [131071, 100003]
    desc, inp, ck, cv, pos_d, mp = _case("full", 2, 131072, "linear", pos1, seed=900)
    print(f"call 1: full layer B=2 cap=131072 pos={pos1}", flush=True)
    _check("call 1", *_run_both(desc, inp, ck, cv, pos_d, mp, "linear"))
    del inp, ck, cv
    torch.cuda.empty_cache()
    # 2: smaller, B = 1 over an 8192-slot linear cache (40 splits), over the
    #    partials call 1 left behind
    pos2 = [5000]
    desc, inp, ck, cv, pos_d, mp = _case("full", 1, 8192, "linear", pos2, seed=910)
    print(f"call 2: full layer B=1 cap=8192 pos={pos2}", flush=True)
    _check("call 2", *_run_both(desc, inp, ck, cv, pos_d, mp, "linear"))


def test_static_scratch_decode_ring_and_single_workgroup_plans():
    # sliding layer on 512-slot rings: B = 3 takes a split plan (12 pairs),
    # B = 64 the one-workgroup-per-pair plan that needs no partials
    for B, seed in ((3, 920), (64, 930)):
        pos = synth.positions_uniform(B, 0, 1 << 20, seed=seed).tolist()
        pos[0] = 17   # a partially filled ring
        desc, inp, ck, cv, pos_d, mp = _case("sliding", B, 512, "ring", pos, seed=seed)
        print(f"ring decode B={B}", flush=True)
        _check(f"ring B={B}", *_run_both(desc, inp, ck, cv, pos_d, mp, "ring"))
