"""kv_attn_decode_compact on the GPU: attention within tolerance of the oracle on the
pre-eviction cache, and the compacted cache bit-exact against the oracle's eviction."""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import (check_attention, check_compacted, check_layout, dev_cache, host_dict, say,
                      snapshot_rows, to_dev, to_host, values)

pytestmark = pytest.mark.gpu


def _setup(seed, B, Hkv, G, D, n, cap, lens=None, retention=True, dtype="bf16"):
    w = synth.Workload("t", batch=B, hq=Hkv * G, hkv=Hkv, head_dim=D, dtype=dtype, ctx=n,
                       budget=0, layers=1, seed=seed, retention=retention)
    d = synth.host_cache(w, n=n, cap=cap)
    if lens is not None:
        d["len"] = np.asarray(lens, np.int32).reshape(B, Hkv)
    rng = np.random.default_rng(seed + 1)
    q = synth.bf16_bits(rng.standard_normal((B, Hkv * G, D)))
    if dtype == "f32":
        q = synth.f32_bits(rng.standard_normal((B, Hkv * G, D)))
    t = (d["len"].max(axis=1) + rng.integers(0, 4, B)).astype(np.int32)
    return d, q, t


def _fused_vs_oracle(d, q, t, M, P, split_phases, what):
    B, H = d["len"].shape
    c = dev_cache(d)
    td = to_dev(t)
    n_ev, wse = kvb.kv_evict_plan(c, td, M)
    if split_phases:
        ws = kvb.kv_attn_decode_workspace(c, q.shape[1], P)
        ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        out, lse = kvb.kv_attn_decode_compact(c, to_dev(q), td, M, wse, num_splits=P, phase=1,
                                              ws=ws)
        out, lse = kvb.kv_attn_decode_compact(c, to_dev(q), td, M, wse, num_splits=P, phase=2,
                                              out=out, lse=lse, ws=ws)
    else:
        out, lse = kvb.kv_attn_decode_compact(c, to_dev(q), td, M, wse, num_splits=P)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_attention(values(d["k"]), values(d["v"]), d["log_beta"],
                                               d["pos"], d["len"], values(q), t)
    check_attention(to_host(out), to_host(lse), ref_out, ref_lse, what)
    ref, _, ref_n = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    check_layout(host_dict(c), ref, what)
    assert np.array_equal(to_host(n_ev), ref_n), f"{what} n_evicted"


@pytest.mark.parametrize("n,cap,M", [(100, 100, 0), (100, 128, 17), (1000, 1001, 100),
                                     (1000, 1004, 256), (4097, 4100, 4096), (5000, 5024, 64),
                                     (9000, 9003, 3000), (20000, 20000, 17), (1000, 1000, 999),
                                     (64, 64, 64), (33, 36, 32)])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_fused_vs_oracle(n, cap, M, G):
    say("fused", n, cap, M, G)
    d, q, t = _setup(n * 3 + M + G, 2, 2, G, 128, n, cap)
    for P in (2, 7, 0):
        _fused_vs_oracle(d, q, t, M, P, False, f"n={n} cap={cap} M={M} G={G} P={P}")


@pytest.mark.parametrize("retention", [True, False])
def test_fused_mixed_lengths_and_phases(retention):
    """Heads above and below the budget in one launch, empty heads, and the two-phase
    form (attention below the destination boundary, then the rest) with one workspace."""
    lens = [[3000, 100, 0, 2500], [1, 2999, 1200, 3000]]
    d, q, t = _setup(77, 2, 4, 2, 128, 3000, 3008, lens=lens, retention=retention)
    for M in (0, 1, 32, 1199, 1200, 2600):
        for split in (False, True):
            _fused_vs_oracle(d, q, t, M, 6, split, f"mixed M={M} split={split} r={retention}")


def test_fused_ties():
    """Equal keys (ties broken by position), log beta = -inf and 0, a slot at the
    decode position."""
    B, H, n = 1, 4, 700
    d, q, t = _setup(5, B, H, 4, 128, n, n)
    lb = d["log_beta"]
    lb[0, 0, :] = np.float32(-0.25)
    lb[0, 1, ::3] = -np.inf
    lb[0, 2, :] = np.where(np.arange(n) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    lb[0, 3, 100:400] = lb[0, 3, 99]
    t = np.array([699], np.int32)
    for M in (0, 50, 350, 699):
        _fused_vs_oracle(d, q, t, M, 4, False, f"ties M={M}")


def test_fused_fallback_paths():
    """float32 caches, head_dim 64 and a single split take the unfused kernels
    through the same entry point; results must still match."""
    for dtype, D, P in (("f32", 128, 4), ("bf16", 64, 4), ("bf16", 128, 1)):
        d, q, t = _setup(11, 1, 2, 4, D, 2000, 2003, dtype=dtype)
        _fused_vs_oracle(d, q, t, 500, P, False, f"fallback {dtype} D={D} P={P}")
        _fused_vs_oracle(d, q, t, 500, P, True, f"fallback split {dtype} D={D} P={P}")


def test_fused_steady_state_loop():
    """Budget M, one token over each step: append, plan, fused attention + compaction
    (every kept row of the first tiles shifts down by one, through the staging list)."""
    B, H, G, D, M = 2, 2, 4, 128, 1000
    d, _, _ = _setup(21, B, H, G, D, M, M + 40)
    c = dev_cache(d)
    ref = oracle.Cache.from_arrays(d)
    rng = np.random.default_rng(5)
    for s in range(8):
        t = np.full(B, M + s, np.int32)
        kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        lbn = np.log(rng.uniform(0.5, 1.0, (B, H))).astype(np.float32)
        qn = synth.bf16_bits(rng.standard_normal((B, G * H, D)))
        td = to_dev(t)
        kvb.kv_append(c, to_dev(kn), to_dev(vn), to_dev(lbn), td)
        _, wse = kvb.kv_evict_plan(c, td, M)
        out, lse = kvb.kv_attn_decode_compact(c, to_dev(qn), td, M, wse, num_splits=5)
        torch.cuda.synchronize()
        oracle.append_tokens(ref, kn, vn, lbn, t)
        ro, rl = oracle.decode_attention(ref.values("k"), ref.values("v"), ref.log_beta, ref.pos,
                                         ref.length, values(qn), t)
        check_attention(to_host(out), to_host(lse), ro, rl, f"steady step {s}")
        ref, _, _ = oracle.evict_to_budget(ref, t, M)
        check_layout(host_dict(c), ref, f"steady step {s}")


def test_fused_tiny_workload_steps():
    """The tiny workload's 16 decode steps through append + plan + fused call."""
    w = synth.WORKLOADS["tiny"]
    d = synth.host_cache(w)
    qs = synth.host_queries(w)
    kn, vn, lbn = synth.host_new_tokens(w)
    c = dev_cache(d)
    ref = oracle.Cache.from_arrays(d)
    for s in range(w.steps):
        t = np.full(w.batch, w.ctx + s, np.int32)
        td = to_dev(t)
        kvb.kv_append(c, to_dev(kn[s]), to_dev(vn[s]), to_dev(lbn[s]), td)
        _, wse = kvb.kv_evict_plan(c, td, w.budget)
        out, lse = kvb.kv_attn_decode_compact(c, to_dev(qs[s]), td, w.budget, wse)
        torch.cuda.synchronize()
        oracle.append_tokens(ref, kn[s], vn[s], lbn[s], t)
        ro, rl = oracle.decode_attention(ref.values("k"), ref.values("v"), ref.log_beta, ref.pos,
                                         ref.length, qs[s].astype(np.float64), t)
        check_attention(to_host(out), to_host(lse), ro, rl, f"tiny step {s}")
        ref, _, _ = oracle.evict_to_budget(ref, t, w.budget)
        check_layout(host_dict(c), ref, f"tiny step {s}")


def test_fused_errors():
    d, q, t = _setup(3, 1, 2, 4, 128, 300, 300)
    c = dev_cache(d)
    td = to_dev(t)
    _, wse = kvb.kv_evict_plan(c, td, 100)
    with pytest.raises(kvb.KVBError):
        kvb.kv_attn_decode_compact(c, to_dev(q), td, 100, wse, phase=3)
    with pytest.raises(kvb.KVBError):
        kvb.kv_attn_decode_compact(c, to_dev(q), td, 100, wse[:16])
    with pytest.raises(kvb.KVBError):
        kvb.kv_attn_decode_compact(c, to_dev(q), td, -1, wse)
    torch.cuda.synchronize()


def test_fused_full_size_qwen3_8b_32k():
    """One full 32K layer as the decode step runs it: append, plan, fused call.
    Attention of sampled heads against the oracle; every head's compacted rows
    against the oracle's plan."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    say("fused full size", w.name)
    dc = synth.device_cache(w, layer=0)
    q, kn, vn, lbn = synth.device_queries(w, 0)
    t = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    c = kvb.KVCache.from_dict(dc)
    kvb.kv_append(c, kn, vn, lbn, t)
    torch.cuda.synchronize()
    n = w.ctx + 1
    G = w.group
    units = [(0, 0), (7, 3), (15, 7)]
    sub = {(b, g): {k: to_host(dc[k][b:b + 1, g:g + 1, :n]) for k in ("k", "v", "log_beta", "pos")}
           for (b, g) in units}
    lbh = to_host(c.log_beta[:, :, :n])
    ph = to_host(c.pos[:, :, :n])
    keep = {}
    for b in range(w.batch):
        for g in range(w.hkv):
            k, _ = oracle.evict_plan(lbh[b, g], ph[b, g], n, w.ctx, w.budget)
            keep[(b, g)] = np.nonzero(k)[0]
    snap = snapshot_rows(c, keep)
    _, wse = kvb.kv_evict_plan(c, t, w.budget)
    out, lse = kvb.kv_attn_decode_compact(c, q, t, w.budget, wse)
    torch.cuda.synchronize()
    check_compacted(c, snap, w.name)
    oh, lh, qh = to_host(out), to_host(lse), to_host(q)
    for (b, g), s in sub.items():
        ro, rl = oracle.decode_attention(values(s["k"]), values(s["v"]), s["log_beta"], s["pos"],
                                         np.array([[n]], np.int32),
                                         values(qh[b:b + 1, g * G:(g + 1) * G]),
                                         np.array([w.ctx]))
        check_attention(oh[b:b + 1, g * G:(g + 1) * G], lh[b:b + 1, g * G:(g + 1) * G], ro, rl,
                        f"{w.name} ({b},{g})")
    del dc, c
    torch.cuda.empty_cache()
