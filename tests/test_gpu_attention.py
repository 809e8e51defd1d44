"""kv_attn_decode on the GPU against the float64 oracle."""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import (check_attention, dev_cache, host_dict, oracle_attention, say, to_dev,
                      to_host, values)

pytestmark = pytest.mark.gpu


def _rand_cache(seed, B, Hkv, n, cap, D, dtype, retention=True, lens=None):
    w = synth.Workload("t", batch=B, hq=Hkv, hkv=Hkv, head_dim=D, dtype=dtype, ctx=n,
                       budget=0, layers=1, seed=seed, retention=retention)
    d = synth.host_cache(w, n=n, cap=cap)
    if lens is not None:
        d["len"] = np.asarray(lens, np.int32).reshape(B, Hkv)
    return d


def _queries(seed, B, Hq, D, dtype):
    w = synth.Workload("t", batch=B, hq=Hq, hkv=1, head_dim=D, dtype=dtype, ctx=1, budget=0,
                       layers=1, seed=seed)
    return synth.host_queries(w, steps=1)[0]


CASES = [
    # B, Hq, Hkv, D, n, dtype, splits
    (1, 4, 1, 128, 1, "bf16", 0),
    (2, 8, 2, 128, 31, "bf16", 0),
    (2, 8, 2, 128, 33, "bf16", 1),
    (1, 32, 8, 128, 1000, "bf16", 0),
    (2, 16, 2, 128, 4097, "bf16", 7),
    (1, 64, 8, 128, 2050, "bf16", 3),     # G = 8
    (2, 4, 2, 128, 300, "bf16", 0),       # G = 2
    (2, 2, 2, 128, 257, "bf16", 0),       # G = 1
    (1, 8, 2, 64, 700, "bf16", 0),        # D = 64
    (1, 16, 2, 64, 129, "bf16", 5),       # D = 64, G = 8
    (1, 6, 2, 128, 200, "bf16", 0),       # G = 3: generic kernel
    (1, 8, 2, 64, 513, "f32", 0),         # float32 generic kernel
    (1, 8, 2, 96, 77, "f32", 3),          # float32, D = 96
]


@pytest.mark.parametrize("retention", [True, False])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_D{}_n{}_{}_P{}".format(*c))
def test_attention_vs_oracle(case, retention):
    B, Hq, Hkv, D, n, dtype, P = case
    say("case", case, retention)
    d = _rand_cache(100 + n, B, Hkv, n, n + 5, D, dtype, retention)
    q = _queries(200 + n, B, Hq, D, dtype)
    t = np.full(B, n + 3, np.int32)       # decode token 3 positions past the last
    c = dev_cache(d)
    out, lse = kvb.kv_attn_decode(c, to_dev(q), to_dev(t), num_splits=P)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_attention(d, q, t)
    check_attention(to_host(out), to_host(lse), ref_out, ref_lse, str(case))


def test_attention_append_then_attend():
    """k_new/v_new/log_beta_new land at slot len with pos = t, then are attended."""
    B, Hq, Hkv, D, n = 2, 8, 2, 128, 100
    d = _rand_cache(7, B, Hkv, n, n + 2, D, "bf16")
    q = _queries(8, B, Hq, D, "bf16")
    kn = synth.bf16_bits(np.random.default_rng(1).standard_normal((B, Hkv, D)))
    vn = synth.bf16_bits(np.random.default_rng(2).standard_normal((B, Hkv, D)))
    lbn = np.full((B, Hkv), -0.5, np.float32)
    t = np.array([n, n + 10], np.int32)
    c = dev_cache(d)
    out, lse = kvb.kv_attn_decode(c, to_dev(q), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                                  log_beta_new=to_dev(lbn))
    torch.cuda.synchronize()
    ref = oracle.Cache.from_arrays(d)
    oracle.append_tokens(ref, kn, vn, lbn, t)
    got = host_dict(c)
    assert got["len"].tolist() == [[n + 1] * Hkv] * B
    for b in range(B):
        for g in range(Hkv):
            assert np.array_equal(got["k"][b, g, n], kn[b, g])
            assert np.array_equal(got["v"][b, g, n], vn[b, g])
            assert got["pos"][b, g, n] == t[b] and got["log_beta"][b, g, n] == lbn[b, g]
    rd = {"k": ref.k, "v": ref.v, "log_beta": ref.log_beta, "pos": ref.pos, "len": ref.length}
    ref_out, ref_lse = oracle_attention(rd, q, t)
    check_attention(to_host(out), to_host(lse), ref_out, ref_lse, "append")


def test_attention_decode_token_full_and_empty_heads():
    """The decode token when a head is full (not appended, not attended, status
    KVB_ECAPACITY) and when a head is empty (its own state is the whole result)."""
    B, Hq, Hkv, D, cap = 1, 8, 4, 128, 64
    d = _rand_cache(17, B, Hkv, cap, cap, D, "bf16")
    d["len"] = np.array([[cap, 0, 5, cap - 1]], np.int32)
    q = _queries(18, B, Hq, D, "bf16")
    rng = np.random.default_rng(19)
    kn = synth.bf16_bits(rng.standard_normal((B, Hkv, D)))
    vn = synth.bf16_bits(rng.standard_normal((B, Hkv, D)))
    lbn = np.full((B, Hkv), -0.25, np.float32)
    t = np.array([cap + 3], np.int32)
    c = dev_cache(d)
    ws = torch.zeros(kvb.kv_attn_decode_workspace(c, Hq), dtype=torch.uint8, device="cuda")
    out, lse = kvb.kv_attn_decode(c, to_dev(q), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                                  log_beta_new=to_dev(lbn), ws=ws)
    torch.cuda.synchronize()
    status = int(to_host(ws[:4]).view(np.int32)[0])
    assert status == -3, f"status {status}: the full head must report KVB_ECAPACITY"
    got = host_dict(c)
    assert got["len"].tolist() == [[cap, 1, 6, cap]]
    ref = oracle.Cache.from_arrays(d)
    for g in range(Hkv):          # the oracle's append, skipping the full head
        s0 = int(ref.length[0, g])
        if s0 < cap:
            ref.k[0, g, s0], ref.v[0, g, s0] = kn[0, g], vn[0, g]
            ref.log_beta[0, g, s0], ref.pos[0, g, s0] = lbn[0, g], t[0]
            ref.length[0, g] = s0 + 1
    rd = {"k": ref.k, "v": ref.v, "log_beta": ref.log_beta, "pos": ref.pos, "len": ref.length}
    ref_out, ref_lse = oracle_attention(rd, q, t)
    check_attention(to_host(out), to_host(lse), ref_out, ref_lse, "full and empty heads")


def test_attention_edges():
    """Empty heads, a single live token, all-but-newest weights zero (log beta = -inf),
    a decode token at the same position as a live slot, more splits than tiles (up
    to the 4096 limit, past the merge's 1024 states held in registers)."""
    B, Hq, Hkv, D, n = 2, 8, 4, 128, 70
    d = _rand_cache(9, B, Hkv, n, n, D, "bf16", lens=[[0, 1, 70, 33], [70, 0, 2, 64]])
    d["log_beta"][0, 2, :] = -np.inf                  # only distance-0 tokens keep weight
    d["log_beta"][1, 3, :] = -np.inf                  # every weight zero -> empty
    q = _queries(10, B, Hq, D, "bf16")
    t = np.array([69, 75], np.int32)                  # b=0: t equals the last live position
    c = dev_cache(d)
    for P in (1, 2, 64, 300, 1100, 4096):
        out, lse = kvb.kv_attn_decode(c, to_dev(q), to_dev(t), num_splits=P)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle_attention(d, q, t)
        check_attention(to_host(out), to_host(lse), ref_out, ref_lse, f"edges P={P}")


def test_attention_deterministic():
    d = _rand_cache(11, 2, 2, 5000, 5000, 128, "bf16")
    q = _queries(12, 2, 8, 128, "bf16")
    t = np.full(2, 5000, np.int32)
    c = dev_cache(d)
    o1, l1 = kvb.kv_attn_decode(c, to_dev(q), to_dev(t))
    o2, l2 = kvb.kv_attn_decode(c, to_dev(q), to_dev(t))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_attention_scale_and_errors():
    d = _rand_cache(13, 1, 2, 64, 64, 128, "bf16")
    q = _queries(14, 1, 8, 128, "bf16")
    t = np.full(1, 64, np.int32)
    c = dev_cache(d)
    out, lse = kvb.kv_attn_decode(c, to_dev(q), to_dev(t), scale=0.3)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_attention(d, q, t, scale=0.3)
    check_attention(to_host(out), to_host(lse), ref_out, ref_lse, "scale")
    with pytest.raises(kvb.KVBError):   # Hq not a multiple of Hkv
        kvb.kv_attn_decode(c, to_dev(q[:, :7].copy()), to_dev(t))
    with pytest.raises(kvb.KVBError):   # workspace too small
        kvb.kv_attn_decode(c, to_dev(q), to_dev(t),
                           ws=torch.empty(300, dtype=torch.uint8, device="cuda"))


def _oracle_unit(w, b, g, s, knh, vnh, lbh, qh):
    """Oracle attention of KV head (b, g)'s query group over its cached tokens with the
    decode token appended (as the call did), from the head's exact input bits."""
    n = w.ctx
    G = w.group
    dd = {"k": np.concatenate([s["k"][:n], knh[b, g][None]])[None, None],
          "v": np.concatenate([s["v"][:n], vnh[b, g][None]])[None, None],
          "log_beta": None if s["log_beta"] is None else
          np.append(s["log_beta"][:n], np.float32(lbh[b, g]))[None, None],
          "pos": np.append(s["pos"][:n], np.int32(w.ctx))[None, None],
          "len": np.array([[n + 1]], np.int32)}
    qs = qh[b:b + 1, g * G:(g + 1) * G]
    return oracle.decode_attention(values(dd["k"]), values(dd["v"]), dd["log_beta"], dd["pos"],
                                   dd["len"], values(qs), np.array([w.ctx]))


def _full_size(w, layer, units, splits_list):
    """Decode attention over one full layer of the workload, with the decode token
    appended by the first call (later calls attend over the same tokens with other
    split counts); every listed KV head's query group against the oracle.  The
    heads' inputs are read back after the calls: they write slot n (the decode
    token) only, which the oracle reconstructs from k_new, v_new."""
    say("full-size", w.name, "layer", layer, "units", len(units), "splits", splits_list)
    dc = synth.device_cache(w, layer)
    q, kn, vn, lbn = synth.device_queries(w, layer)
    t = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    G = w.group
    qh = to_host(q)
    knh, vnh = to_host(kn), to_host(vn)
    lbh = to_host(lbn) if lbn is not None else None
    c = kvb.KVCache.from_dict(dc)
    outs = []
    for i, P in enumerate(splits_list):
        if i == 0:
            out, lse = kvb.kv_attn_decode(c, q, t, k_new=kn, v_new=vn, log_beta_new=lbn,
                                          num_splits=P)
        else:
            out, lse = kvb.kv_attn_decode(c, q, t, num_splits=P)
        torch.cuda.synchronize()
        outs.append((P, to_host(out), to_host(lse)))
    worst = 0.0
    for j, (b, g) in enumerate(units):
        s = {k: to_host(dc[k][b, g]) if dc[k] is not None else None
             for k in ("k", "v", "log_beta", "pos")}
        ref_out, ref_lse = _oracle_unit(w, b, g, s, knh, vnh, lbh, qh)
        for P, oh, lh in outs:
            worst = max(worst, check_attention(oh[b:b + 1, g * G:(g + 1) * G],
                                               lh[b:b + 1, g * G:(g + 1) * G], ref_out, ref_lse,
                                               f"{w.name} layer {layer} ({b},{g}) P={P}"))
        if j % 32 == 31:
            say("  checked", j + 1, "heads")
    say("  worst relative error", worst)
    del dc, c
    torch.cuda.empty_cache()


def test_attention_full_size_qwen3_8b_32k():
    """Every KV head (all 128 query groups) of a 32K layer at the default split
    count, and at 128 splits."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    _full_size(w, 0, [(b, g) for b in range(w.batch) for g in range(w.hkv)], [0, 128])


def test_attention_full_size_qwen3_32b_128k():
    """Eight KV heads (64 query heads) of each of two 128K layers, at the default
    split count and at 64, 128 and 256 splits."""
    w = synth.WORKLOADS["qwen3_32b_128k"]
    rng = np.random.default_rng(5)
    for layer in (0, 37):
        units = sorted(set((int(b), int(g)) for b, g in
                           zip(rng.integers(0, w.batch, 40), rng.integers(0, w.hkv, 40))))[:8]
        _full_size(w, layer, units, [0, 64, 128, 256])
