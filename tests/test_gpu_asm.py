"""asm_lookup_merge on the GPU against the float64 oracle.

Index parity: the GPU index equals the oracle's, or -- at a near-tie, where float32
rounding may pick another centroid -- its true cosine is within 1e-5 of the best
(an fp32 error bound for D = 128 dot products); the merged output is then checked
against the oracle merge at the GPU's index.
"""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import check_attention, dev_cache, say, to_dev, to_host, values

pytestmark = pytest.mark.gpu
COS_TOL = 1e-5


def _check_asm(qh, ch, ah, lzh, so, sl, out, lse, idx, what):
    B, Hq, D = qh.shape
    Hkv = ch.shape[0]
    G = Hq // Hkv
    qv, cv = values(qh), values(ch)
    ref_idx = np.zeros((B, Hq), np.int32)
    use_idx = np.zeros((B, Hq), np.int32)
    ties = 0
    for b in range(B):
        for h in range(Hq):
            g = h // G
            cos = oracle.cosine_similarities(qv[b, h], cv[g])
            ri = int(np.argmax(cos))
            ref_idx[b, h] = ri
            gi = int(idx[b, h])
            if gi != ri:
                assert 0 <= gi < cv.shape[1], f"{what} idx out of range"
                assert cos[gi] >= cos[ri] - COS_TOL, f"{what} ({b},{h}) idx {gi} vs {ri}"
                ties += 1
            use_idx[b, h] = gi
    ro = np.zeros((B, Hq, D))
    rl = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            k = use_idx[b, h]
            ro[b, h], rl[b, h] = oracle.asm_merge(so[b, h], sl[b, h], values(ah[g, k]),
                                                  float(lzh[g, k]))
    check_attention(out, lse, ro, rl, what)
    return ties


def test_asm_full_size_layer():
    """One layer of the ASM workload: self-attention over 2048 generated tokens
    (beta == 1), then lookup in a 4096-entry codebook per KV head and merge."""
    w = synth.WORKLOADS["asm_lookup"]
    say("asm full size")
    dc = synth.device_cache(w, layer=0, n=w.ctx, cap=w.ctx)
    q, _, _, _ = synth.device_queries(w, 0)
    cent, abar, lz = synth.device_codebook(w, 0)
    c = kvb.KVCache.from_dict(dc)
    t = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    so, sl = kvb.kv_attn_decode(c, q, t)
    out, lse, idx = kvb.asm_lookup_merge(q, cent, abar, lz, so, sl)
    torch.cuda.synchronize()
    qh, ch, ah, lzh = to_host(q), to_host(cent), to_host(abar), to_host(lz)
    soh, slh = to_host(so), to_host(sl)
    # the self state itself against the oracle (sampled heads)
    kh, vh, ph = to_host(dc["k"][:4]), to_host(dc["v"][:4]), to_host(dc["pos"][:4])
    ro, rl = oracle.decode_attention(values(kh), values(vh), None, ph,
                                     np.full((4, w.hkv), w.ctx), values(qh[:4]),
                                     np.full(4, w.ctx))
    check_attention(soh[:4], slh[:4], ro, rl, "asm self attention")
    ties = _check_asm(qh, ch, ah, lzh, soh, slh, to_host(out), to_host(lse), to_host(idx),
                      "asm layer")
    say("near-ties", ties)


def test_asm_small_edges():
    """K = 1; duplicate centroids (lowest index wins); a zero query (index 0);
    log Zbar = -inf (own state unchanged); self_lse = -inf (stored state)."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, D = 3, 8, 2, 128
    for K in (1, 5, 17, 1500):
        qh = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
        cf = rng.standard_normal((Hkv, K, D))
        if K >= 5:
            cf[:, 4] = cf[:, 2]                           # duplicate rows
            qh[0, 0] = synth.bf16_bits(cf[0, 2] * 3.0)     # exact direction of a duplicate
        ch = synth.bf16_bits(cf)
        ah = synth.bf16_bits(rng.standard_normal((Hkv, K, D)))
        lzh = rng.uniform(0, 12, (Hkv, K)).astype(np.float32)
        lzh[1, 0] = -np.inf
        qh[2, 3] = 0                                       # zero query
        so = rng.standard_normal((B, Hq, D)).astype(np.float32)
        sl = rng.uniform(-5, 15, (B, Hq)).astype(np.float32)
        sl[1, 1] = -np.inf
        out, lse, idx = kvb.asm_lookup_merge(to_dev(qh), to_dev(ch), to_dev(ah), to_dev(lzh),
                                             to_dev(so), to_dev(sl))
        torch.cuda.synchronize()
        idxh = to_host(idx)
        assert idxh[2, 3] == 0, "zero query -> index 0"
        if K >= 5:
            assert idxh[0, 0] == 2, "duplicate centroid: lowest index"
        _check_asm(qh, ch, ah, lzh, so, sl, to_host(out), to_host(lse), idxh, f"asm K={K}")


def _fused_vs_two_calls(c_two, c_fused, q, t, cent, abar, lz, kn=None, vn=None, splits=0):
    """kv_attn_decode + asm_lookup_merge on one cache, kv_attn_decode_asm on an
    identical one: every output bit-equal, and the caches (appended rows) too.  With
    splits 0 the fused entry takes its own default, which the two calls are given."""
    two = splits or kvb.kv_attn_decode_asm_splits(c_two, q.shape[1], cent.shape[1])
    so, sl = kvb.kv_attn_decode(c_two, q, t, k_new=kn, v_new=vn, num_splits=two)
    so_h, sl_h = to_host(so), to_host(sl)
    out2, lse2, idx2 = kvb.asm_lookup_merge(q, cent, abar, lz, so, sl)
    out1, lse1, idx1 = kvb.kv_attn_decode_asm(c_fused, q, t, cent, abar, lz, k_new=kn, v_new=vn,
                                              num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2), "fused lookup index"
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2), "fused merged state"
    assert torch.equal(c_two.length, c_fused.length)
    for name in ("k", "v", "pos"):
        assert torch.equal(getattr(c_two, name), getattr(c_fused, name)), name
    return so_h, sl_h, out1, lse1, idx1


def test_attn_decode_asm_full_size_layer():
    """One layer of the ASM workload through the fused entry (decode token appended,
    self-attention over 2049 tokens, lookup, merge) equals the two calls, and the
    merged state matches the oracle merge of the self state."""
    w = synth.WORKLOADS["asm_lookup"]
    say("fused asm full size")
    d1 = synth.device_cache(w, layer=0)
    d2 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d1.items()}
    q, kn, vn, _ = synth.device_queries(w, 0)
    cent, abar, lz = synth.device_codebook(w, 0)
    t = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    so, sl, out, lse, idx = _fused_vs_two_calls(kvb.KVCache.from_dict(d1),
                                                kvb.KVCache.from_dict(d2), q, t, cent, abar, lz,
                                                kn, vn)
    ties = _check_asm(to_host(q), to_host(cent), to_host(abar), to_host(lz), so, sl,
                      to_host(out), to_host(lse), to_host(idx), "fused asm layer")
    say("near-ties", ties)


@pytest.mark.parametrize("D", [128, 64])
def test_attn_decode_asm_edges(D):
    """Fused entry on small caches: an empty head, a zero query (entry 0), log Zbar =
    -inf entries, K not a multiple of the lookup chunk, a split count above the
    tile count; equal to the two calls and to the oracle merge."""
    rng = np.random.default_rng(D)
    B, Hq, Hkv, K = 2, 8, 2, 300
    n = 90
    w = synth.Workload("t", batch=B, hq=Hkv, hkv=Hkv, head_dim=D, dtype="bf16", ctx=n,
                       budget=0, layers=1, seed=7, retention=False)
    d = synth.host_cache(w, n=n, cap=n + 4)
    d["len"] = np.array([[90, 0], [33, 61]], np.int32)
    qh = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
    qh[1, 5] = 0
    ch = synth.bf16_bits(rng.standard_normal((Hkv, K, D)))
    ah = synth.bf16_bits(rng.standard_normal((Hkv, K, D)))
    lzh = rng.uniform(0, 12, (Hkv, K)).astype(np.float32)
    lzh[:, ::7] = -np.inf
    t = np.array([n + 2, n + 9], np.int32)
    for splits in (0, 11):
        so, sl, out, lse, idx = _fused_vs_two_calls(dev_cache(d), dev_cache(d), to_dev(qh),
                                                    to_dev(t), to_dev(ch), to_dev(ah),
                                                    to_dev(lzh), splits=splits)
        idxh = to_host(idx)
        assert idxh[1, 5] == 0, "zero query -> index 0"
        _check_asm(qh, ch, ah, lzh, so, sl, to_host(out), to_host(lse), idxh,
                   f"fused edges D={D} P={splits}")


def test_attn_decode_asm_graph_and_user_stream():
    """kv_attn_decode_asm over three layers sharing one workspace, launched on a
    user stream: eagerly, and captured in one HIP graph replayed three times with new
    queries written (and other eager work and synchronisations) in between; every
    result equals the two-call path on the same inputs."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D, K, n, L = 4, 16, 4, 128, 1000, 700, 3
    w = synth.Workload("t", batch=B, hq=Hkv, hkv=Hkv, head_dim=D, dtype="bf16", ctx=n,
                       budget=0, layers=1, seed=5, retention=False)
    hosts = [synth.host_cache(w, n=n, cap=n + 8) for _ in range(L)]
    for h in hosts:
        h["len"] = rng.integers(n - 300, n + 1, (B, Hkv)).astype(np.int32)
    books = [tuple(to_dev(x) for x in (
        synth.bf16_bits(rng.standard_normal((Hkv, K, D))),
        synth.bf16_bits(rng.standard_normal((Hkv, K, D))),
        rng.uniform(0, 12, (Hkv, K)).astype(np.float32))) for _ in range(L)]
    t = to_dev(np.full(B, n + 3, np.int32))
    caches = [dev_cache(h) for h in hosts]
    q = torch.empty((L, B, Hq, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((L, B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, B, Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((L, B, Hq), dtype=torch.int32, device="cuda")
    ws = torch.empty(kvb.kv_attn_decode_asm_workspace(caches[0], Hq, 0, K), dtype=torch.uint8,
                     device="cuda")
    user = torch.cuda.Stream()

    def layers():
        for i in range(L):
            kvb.kv_attn_decode_asm(caches[i], q[i], t, *books[i], out=out[i], lse=lse[i],
                                   idx=idx[i], ws=ws, stream=user)

    def expect():
        res = []
        for i in range(L):
            so, sl = kvb.kv_attn_decode(caches[i], q[i], t)
            res.append(kvb.asm_lookup_merge(q[i], *books[i], so, sl))
        torch.cuda.synchronize()
        return res

    def compare(what):
        for i, (o2, l2, i2) in enumerate(expect()):
            assert torch.equal(idx[i], i2), f"{what} layer {i} index"
            assert torch.equal(out[i], o2) and torch.equal(lse[i], l2), f"{what} layer {i}"

    def new_queries():
        q.copy_(to_dev(synth.bf16_bits(rng.standard_normal((L, B, Hq, D)))).view(q.shape))

    say("fused asm eager on a user stream")
    new_queries()
    torch.cuda.synchronize()
    layers()
    user.synchronize()
    compare("eager")
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(user):
        with torch.cuda.graph(graph, stream=user):
            layers()
    torch.cuda.synchronize()
    for r in range(3):
        say("fused asm graph replay", r)
        new_queries()
        out.fill_(float("nan"))
        idx.fill_(-1)
        torch.cuda.synchronize()
        with torch.cuda.stream(user):
            graph.replay()
        user.synchronize()
        compare(f"replay {r}")
