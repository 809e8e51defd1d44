"""kv_attn_decode_noalloc (no workspace, device-resident scratch) against
kv_attn_decode (caller workspace) through the C ABI.

Two calls in a row, the second on a smaller cache, each compared bit for bit with
the workspace entry point on identical copies of the cache (same kernels, same
split count), and with the float64 oracle to the attention tolerance; then a full
head (status word KVB_ECAPACITY) followed by a call that must reset it.
"""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import check_attention, dev_cache, host_dict, say, to_dev, to_host

pytestmark = pytest.mark.gpu

KVB_ECAPACITY = -3


def _inputs(seed, B, Hq, Hkv, D, n, cap, dtype="bf16"):
    w = synth.Workload("t", batch=B, hq=Hq, hkv=Hkv, head_dim=D, dtype=dtype, ctx=n,
                       budget=0, layers=1, seed=seed, retention=True)
    d = synth.host_cache(w, n=n, cap=cap)
    q = synth.host_queries(w, steps=1)[0]
    kn, vn, lbn = synth.host_new_tokens(w, steps=1)
    t = np.full(B, n, np.int32)
    return d, q, kn[0], vn[0], lbn[0], t


def _pair(d, q, kn, vn, lbn, t, P):
    """Both entry points on identical device copies of one cache."""
    ca, cb = dev_cache(d), dev_cache(d)
    qd, td = to_dev(q), to_dev(t)
    B, Hq, D = q.shape
    ws = torch.zeros(kvb.kv_attn_decode_workspace(ca, Hq, P), dtype=torch.uint8, device="cuda")
    oa, la = kvb.kv_attn_decode(ca, qd, td, k_new=to_dev(kn), v_new=to_dev(vn),
                                log_beta_new=to_dev(lbn), num_splits=P, ws=ws)
    ob = torch.full((B, Hq, D), np.nan, dtype=torch.float32, device="cuda")
    lb = torch.full((B, Hq), np.nan, dtype=torch.float32, device="cuda")
    st = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    kvb.kv_attn_decode_noalloc(cb, qd, td, ob, lb, k_new=to_dev(kn), v_new=to_dev(vn),
                               log_beta_new=to_dev(lbn), num_splits=P, status=st)
    torch.cuda.synchronize()
    return ca, cb, oa, la, ob, lb, kvb.workspace_status(ws), int(st.item())


def _compare(what, d, q, kn, vn, lbn, t, P):
    say("noalloc", what, "P", P, "B,Hq,D", q.shape, "n", int(d["len"].max()))
    ca, cb, oa, la, ob, lb, st_ws, st_na = _pair(d, q, kn, vn, lbn, t, P)
    assert st_ws == 0 and st_na == 0, (st_ws, st_na)
    assert np.array_equal(to_host(oa).view(np.uint32), to_host(ob).view(np.uint32)), what
    assert np.array_equal(to_host(la).view(np.uint32), to_host(lb).view(np.uint32)), what
    ha, hb = host_dict(ca), host_dict(cb)
    for k in ("k", "v", "log_beta", "pos", "len"):
        assert np.array_equal(np.asarray(ha[k]).view(np.uint8), np.asarray(hb[k]).view(np.uint8)), k
    ref = oracle.Cache.from_arrays(d)
    oracle.append_tokens(ref, kn, vn, lbn, t)
    ro, rl = oracle.decode_attention(ref.values("k"), ref.values("v"), ref.log_beta, ref.pos,
                                     ref.length, q.astype(np.float64) if q.dtype != np.uint16
                                     else (q.astype(np.uint32) << 16).view(np.float32)
                                     .astype(np.float64), t)
    check_attention(to_host(ob), to_host(lb), ro, rl, what)


def test_noalloc_two_calls_second_smaller():
    # first call: 4 sequences x 8 KV heads x 4 query heads, 3000 tokens, auto splits
    d, q, kn, vn, lbn, t = _inputs(71, 4, 32, 8, 128, 3000, 3008)
    _compare("first", d, q, kn, vn, lbn, t, 0)
    # second call, smaller: fewer sequences, heads, tokens and splits; ragged lengths
    d, q, kn, vn, lbn, t = _inputs(72, 2, 8, 2, 128, 500, 520)
    d["len"] = np.array([[500, 137], [1, 499]], np.int32)
    _compare("second (smaller)", d, q, kn, vn, lbn, t, 3)
    # a float32 cache (generic kernel), smaller again
    d, q, kn, vn, lbn, t = _inputs(73, 1, 8, 2, 64, 77, 80, "f32")
    _compare("float32", d, q, kn, vn, lbn, t, 2)


def test_noalloc_status_word_is_per_call():
    d, q, kn, vn, lbn, t = _inputs(74, 2, 8, 2, 128, 64, 64)   # every head full
    say("noalloc full heads")
    _, _, _, _, _, _, st_ws, st_na = _pair(d, q, kn, vn, lbn, t, 2)
    assert st_ws == KVB_ECAPACITY and st_na == KVB_ECAPACITY, (st_ws, st_na)
    d, q, kn, vn, lbn, t = _inputs(75, 1, 4, 1, 128, 30, 40)   # room again: reset to OK
    _compare("after a full call", d, q, kn, vn, lbn, t, 0)


def test_noalloc_rejects_calls_beyond_its_scratch():
    B, Hq, Hkv, D, cap = 64, 64, 8, 128, 8192
    c = kvb.KVCache(torch.zeros((B, Hkv, cap, D), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((B, Hkv, cap, D), dtype=torch.bfloat16, device="cuda"), None,
                    torch.zeros((B, Hkv, cap), dtype=torch.int32, device="cuda"),
                    torch.zeros((B, Hkv), dtype=torch.int32, device="cuda"))
    assert kvb.kv_attn_decode_workspace(c, Hq, 32) > kvb.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    with pytest.raises(kvb.KVBError) as e:
        kvb.kv_attn_decode_noalloc(c, q, t, out, lse, num_splits=32)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert not out.any() and not lse.any()
