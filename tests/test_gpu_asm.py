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
