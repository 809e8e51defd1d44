"""Latent memory of evicted tokens on the GPU against the float64 oracle.

kv_latent_absorb between kv_evict_plan and kv_evict_apply must equal the oracle's
sequential decayed accumulation over exactly the tokens the oracle evicts (the
eviction itself is bit-exact); tolerance 1e-5 of the state's largest entry (phi(k)
enters the matrix product as two bf16 parts, sums in float32).  Heads with nothing
evicted keep their state bit for bit.  kv_latent_read against the oracle read of
the GPU's state, 1e-5 relative.
"""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import dev_cache, say, to_dev, to_host, values

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _cache(seed, B, Hkv, n, cap, D, lens=None):
    w = synth.Workload("l", batch=B, hq=Hkv, hkv=Hkv, head_dim=D, dtype="bf16", ctx=n,
                       budget=0, layers=1, seed=seed, retention=True)
    d = synth.host_cache(w, n=n, cap=cap)
    if lens is not None:
        d["len"] = np.asarray(lens, np.int32).reshape(B, Hkv)
    return d


def _ref_absorb(d, t, M, lam, M0, b0):
    B, H = d["len"].shape
    RM, Rb, nev = M0.astype(np.float64).copy(), b0.astype(np.float64).copy(), np.zeros((B, H), int)
    for b in range(B):
        for g in range(H):
            n = int(d["len"][b, g])
            keep, _ = oracle.evict_plan(d["log_beta"][b, g], d["pos"][b, g], n, int(t[b]), M)
            K = values(d["k"][b, g, :n][~keep])
            V = values(d["v"][b, g, :n][~keep])
            nev[b, g] = K.shape[0]
            RM[b, g], Rb[b, g] = oracle.latent_absorb(RM[b, g], Rb[b, g], K, V, lam)
    return RM, Rb, nev


def _gpu_absorb(d, t, M, lam, M0, b0):
    c = dev_cache(d)
    mM, mb = to_dev(M0.astype(np.float32)), to_dev(b0.astype(np.float32))
    _, ws_e = kvb.kv_evict_plan(c, to_dev(np.asarray(t, np.int32)), M)
    kvb.kv_latent_absorb(c, M, ws_e, lam, mM, mb)
    kvb.kv_evict_apply(c, M, ws_e)
    torch.cuda.synchronize()
    return c, to_host(mM), to_host(mb)


def _check_state(gM, gb, RM, Rb, M0, b0, nev, what):
    B, H = nev.shape
    for b in range(B):
        for g in range(H):
            if nev[b, g] == 0:
                assert np.array_equal(gM[b, g].view(np.uint32),
                                      M0[b, g].astype(np.float32).view(np.uint32)), \
                    f"{what} ({b},{g}) state changed with nothing evicted"
                assert np.array_equal(gb[b, g].view(np.uint32),
                                      b0[b, g].astype(np.float32).view(np.uint32))
                continue
            sM = max(np.abs(RM[b, g]).max(), 1e-30)
            sb = max(np.abs(Rb[b, g]).max(), 1e-30)
            eM = np.abs(gM[b, g] - RM[b, g]).max() / sM
            eb = np.abs(gb[b, g] - Rb[b, g]).max() / sb
            assert eM <= TOL and eb <= TOL, f"{what} ({b},{g}) M err {eM:.2e} b err {eb:.2e}"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n,M,lam", [(5, 3, 0.9), (100, 99, 0.5), (513, 256, 1.0),
                                     (4097, 4096, 0.999), (9000, 700, 0.9999),
                                     (20000, 17, 0.99995), (300, 300, 0.9)])
def test_absorb_vs_oracle(D, n, M, lam):
    say("latent absorb", D, n, M, lam)
    lam = float(np.float32(lam))
    B, H = 2, 3
    d = _cache(n + M + D, B, H, n, n + 5, D, lens=[[n, n, max(1, n // 2)], [n, n - 1, n]])
    t = np.array([n, n + 3], np.int32)
    rng = np.random.default_rng(n)
    M0 = rng.standard_normal((B, H, D, D)).astype(np.float32)
    b0 = np.abs(rng.standard_normal((B, H, D))).astype(np.float32)
    RM, Rb, nev = _ref_absorb(d, t, M, lam, M0, b0)
    _, gM, gb = _gpu_absorb(d, t, M, lam, M0, b0)
    _check_state(gM, gb, RM, Rb, M0, b0, nev, f"D{D} n{n} M{M}")


def test_absorb_large_cache_plan():
    """A cache too large for the planner's LDS path (45,000 slots): the evicted
    slots come from the plan's kept list instead of its per-tile masks."""
    say("latent absorb, large cache")
    B, H, D, n, M = 1, 2, 128, 45000, 4000
    lam = float(np.float32(0.99995))
    d = _cache(91, B, H, n, n + 7, D, lens=[[n, n - 3000]])
    t = np.array([n], np.int32)
    rng = np.random.default_rng(9)
    M0 = rng.standard_normal((B, H, D, D)).astype(np.float32)
    b0 = np.abs(rng.standard_normal((B, H, D))).astype(np.float32)
    RM, Rb, nev = _ref_absorb(d, t, M, lam, M0, b0)
    _, gM, gb = _gpu_absorb(d, t, M, lam, M0, b0)
    _check_state(gM, gb, RM, Rb, M0, b0, nev, "large cache")


def test_absorb_steps_then_read():
    """Several decode steps (append, evict 1..2, absorb), then the read-out added to
    the attention output; checked against the oracle at every step."""
    B, H, Hq, D, n, M = 2, 2, 8, 128, 600, 596
    d = _cache(5, B, H, n, n + 16, D)
    w = synth.Workload("l", batch=B, hq=Hq, hkv=H, head_dim=D, dtype="bf16", ctx=n, budget=M,
                       layers=1, seed=5, retention=True)
    kn, vn, lbn = synth.host_new_tokens(w, steps=4)
    qs = synth.host_queries(w, steps=4)
    prm = synth.host_latent_params(D, Hq, 77)
    lam = prm["lam"]
    c = dev_cache(d)
    ref = oracle.Cache.from_arrays(d)
    RM = np.zeros((B, H, D, D))
    Rb = np.zeros((B, H, D))
    mM = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    mb = torch.zeros((B, H, D), dtype=torch.float32, device="cuda")
    W_o, w_g, c_g = (to_dev(prm[k]) for k in ("W_o", "w_g", "c_g"))
    for s in range(4):
        t = np.full(B, n + s, np.int32)
        td = to_dev(t)
        out, lse = kvb.kv_attn_decode(c, to_dev(qs[s]), td, k_new=to_dev(kn[s]),
                                      v_new=to_dev(vn[s]), log_beta_new=to_dev(lbn[s]))
        _, ws_e = kvb.kv_evict_plan(c, td, M)
        kvb.kv_latent_absorb(c, M, ws_e, lam, mM, mb)
        kvb.kv_evict_apply(c, M, ws_e)
        o2 = out.clone()
        kvb.kv_latent_read(to_dev(qs[s]), mM, mb, W_o, w_g, c_g, prm["eps"], o2)
        torch.cuda.synchronize()
        oracle.append_tokens(ref, kn[s], vn[s], lbn[s], t)
        for b in range(B):
            for g in range(H):
                nn = int(ref.length[b, g])
                keep, _ = oracle.evict_plan(ref.log_beta[b, g], ref.pos[b, g], nn, int(t[b]), M)
                RM[b, g], Rb[b, g] = oracle.latent_absorb(
                    RM[b, g], Rb[b, g], ref.values("k")[b, g, :nn][~keep],
                    ref.values("v")[b, g, :nn][~keep], lam)
        ref, _, _ = oracle.evict_to_budget(ref, t, M)
        gM, gb = to_host(mM), to_host(mb)
        _check_state(gM, gb, RM, Rb, np.zeros_like(gM), np.zeros_like(gb),
                     np.ones((B, H), int), f"step {s}")
        oh, o2h = to_host(out), to_host(o2)
        qv = values(qs[s])
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // H)
                want = oracle.latent_residual(oh[b, h], gM[b, g], gb[b, g], qv[b, h],
                                              prm["W_o"], prm["w_g"][h], prm["c_g"][h],
                                              prm["eps"])
                err = np.abs(o2h[b, h] - want).max() / max(np.abs(want).max(), 1e-30)
                assert err <= TOL, f"step {s} read ({b},{h}) err {err:.2e}"


@pytest.mark.parametrize("D", [64, 128])
def test_read_vs_oracle(D):
    """Read-out alone on random states (b > 0), G = 1, 4 and 8 query heads per KV head."""
    rng = np.random.default_rng(D)
    for B, Hq, Hkv in ((3, 4, 4), (2, 16, 4), (1, 8, 1)):
        Mst = rng.standard_normal((B, Hkv, D, D)).astype(np.float32)
        bst = (np.abs(rng.standard_normal((B, Hkv, D))) + 0.1).astype(np.float32)
        q = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
        prm = synth.host_latent_params(D, Hq, D + Hq)
        o = rng.standard_normal((B, Hq, D)).astype(np.float32)
        out = to_dev(o.copy())
        kvb.kv_latent_read(to_dev(q), to_dev(Mst), to_dev(bst), to_dev(prm["W_o"]),
                           to_dev(prm["w_g"]), to_dev(prm["c_g"]), prm["eps"], out)
        torch.cuda.synchronize()
        got = to_host(out)
        qv = values(q)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                want = oracle.latent_residual(o[b, h], Mst[b, g], bst[b, g], qv[b, h],
                                              prm["W_o"], prm["w_g"][h], prm["c_g"][h],
                                              prm["eps"])
                err = np.abs(got[b, h] - want).max() / max(np.abs(want).max(), 1e-30)
                assert err <= TOL, f"read D{D} ({b},{h}) err {err:.2e}"


def test_absorb_full_size_sampled():
    """The 32K decode workload's first layer: eviction of 28,673 tokens per KV head
    absorbed from a zero state; two heads checked against the oracle."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    say("latent full size")
    dc = synth.device_cache(w, layer=0)
    c = kvb.KVCache.from_dict(dc)
    M = w.budget
    D = w.head_dim
    t = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    lam = float(np.float32(0.9999))
    mM = torch.zeros((w.batch, w.hkv, D, D), dtype=torch.float32, device="cuda")
    mb = torch.zeros((w.batch, w.hkv, D), dtype=torch.float32, device="cuda")
    units = [(0, 0), (11, 5)]
    host = {u: {k: to_host(dc[k][u[0], u[1]]) for k in ("k", "v", "log_beta", "pos")}
            for u in units}
    lens = to_host(dc["len"])
    _, ws_e = kvb.kv_evict_plan(c, t, M)
    kvb.kv_latent_absorb(c, M, ws_e, lam, mM, mb)
    torch.cuda.synchronize()
    gM, gb = to_host(mM), to_host(mb)
    for (b, g) in units:
        h = host[(b, g)]
        n = int(lens[b, g])
        keep, _ = oracle.evict_plan(h["log_beta"], h["pos"], n, w.ctx, M)
        RM, Rb = oracle.latent_absorb(np.zeros((D, D)), np.zeros(D), values(h["k"][:n][~keep]),
                                      values(h["v"][:n][~keep]), lam)
        eM = np.abs(gM[b, g] - RM).max() / np.abs(RM).max()
        eb = np.abs(gb[b, g] - Rb).max() / np.abs(Rb).max()
        say("full size", b, g, "evicted", int((~keep).sum()), "errors", eM, eb)
        assert eM <= TOL and eb <= TOL
    del dc, c
    torch.cuda.empty_cache()
