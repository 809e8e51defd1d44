"""kv_evict_to_budget / kv_erase_ranges on the GPU: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import (check_attention, check_compacted, check_layout, dev_cache, host_dict, say,
                      snapshot_rows, to_dev, to_host, values)

pytestmark = pytest.mark.gpu


def _cache(seed, B, Hkv, n, cap, D, dtype="bf16", retention=True, lens=None):
    w = synth.Workload("t", batch=B, hq=Hkv, hkv=Hkv, head_dim=D, dtype=dtype, ctx=n,
                       budget=0, layers=1, seed=seed, retention=retention)
    d = synth.host_cache(w, n=n, cap=cap)
    if lens is not None:
        d["len"] = np.asarray(lens, np.int32).reshape(B, Hkv)
    return d


def _evict_and_check(d, t, M, what, max_evict=None):
    B, H = d["len"].shape
    n_max = int(d["len"].max())
    c = dev_cache(d)
    me = max_evict if max_evict is not None else max(1, n_max)
    ev = torch.full((B, H, me), -7, dtype=torch.int32, device="cuda")
    n_ev = kvb.kv_evict_to_budget(c, to_dev(np.asarray(t, np.int32)), M, evicted_pos=ev)
    torch.cuda.synchronize()
    ref, ref_ev, ref_n = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    check_layout(host_dict(c), ref, what)
    assert np.array_equal(to_host(n_ev), ref_n), f"{what} n_evicted"
    evh = to_host(ev)
    for b in range(B):
        for g in range(H):
            k = min(int(ref_n[b, g]), me)
            assert np.array_equal(evh[b, g, :k], ref_ev[b][g][:k]), f"{what} ({b},{g}) evicted_pos"
    return c, ref


@pytest.mark.parametrize("n,M", [(1, 0), (1, 1), (5, 3), (33, 32), (100, 0), (100, 99),
                                 (513, 256), (4097, 4096), (5000, 64), (10000, 9000),
                                 (20000, 17)])
@pytest.mark.parametrize("retention", [True, False])
def test_evict_vs_oracle(n, M, retention):
    say("evict", n, M, retention)
    d = _cache(n * 7 + M, 2, 3, n, n + 3, 128, retention=retention)
    t = np.array([n, n + 5], np.int32)
    _evict_and_check(d, t, M, f"n={n} M={M} r={retention}")


def test_evict_ties_and_special_keys():
    """Equal keys (ties by position), log beta = -inf, log beta = 0 and -0.0,
    a live slot at the decode position, n <= M heads left untouched."""
    B, H, n = 1, 6, 300
    d = _cache(3, B, H, n, n, 128, lens=[[300, 300, 300, 300, 300, 100]])
    lb = d["log_beta"]
    lb[0, 0, :] = np.float32(-0.25)               # one shared beta: sliding window
    lb[0, 1, ::3] = -np.inf                        # weight-zero tokens go first
    lb[0, 2, :] = np.where(np.arange(n) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    lb[0, 3, 50:60] = np.float32(-1e-30)           # tiny keys
    lb[0, 4, :] = np.float32(-0.001)
    lb[0, 4, 100:200] = lb[0, 4, 99]               # long run of equal log beta
    t = np.array([299], np.int32)                  # pos 299 sits at distance 0
    for M in (0, 1, 50, 150, 299):
        _evict_and_check(d, t, M, f"ties M={M}")


def test_evict_one_float32_tie_cluster():
    """One eviction (n = M + 1, the planner's reduction path) whose minimum sits in a
    cluster of keys that round to the same float32 value but differ as doubles
    (lb_i = fl32(c / d_i)); equal exact minima at two slots (the lower goes); every
    key equal; -inf keys."""
    B, H, n = 1, 4, 5000
    d = _cache(7, B, H, n, n + 3, 128)
    lb = d["log_beta"]
    t = np.array([n + 5], np.int32)
    dist = (t[0] - np.arange(n)).astype(np.float64)
    cl = np.arange(1000, 3000)
    lb[0, 0, :n] = np.float32(-0.5)                 # far from the cluster's keys
    lb[0, 0, cl] = (-7.0 / dist[cl]).astype(np.float32)
    keys = dist * lb[0, 0, :n].astype(np.float64)
    assert len(np.unique(keys[cl].astype(np.float32))) < len(np.unique(keys[cl]))
    lb[0, 1, :n] = np.float32(-0.25)
    lb[0, 1, 1005] = np.float32(-5.0)                # d = 4000: key -20000
    lb[0, 1, 3005] = np.float32(-10.0)               # d = 2000: key -20000 (exact tie)
    lb[0, 2, :n] = np.float32(0.0)                   # all keys 0: the oldest goes
    lb[0, 3, :n] = np.float32(-0.1)
    lb[0, 3, [7, 4000, 4500]] = -np.inf              # the first -inf goes
    _evict_and_check(d, t, n - 1, "one eviction")


@pytest.mark.parametrize("n", [5000, 40000])
def test_evict_subnormal_and_far_keys(n):
    """Keys whose float32 rounding is subnormal (subnormal log beta, or tiny log
    beta times a distance), distances above 2^24 (beyond which the float32 key is
    rounded from the double product), on the LDS planner (5000 slots) and on the
    chunked selection (40000)."""
    B, H = 2, 2
    d = _cache(11 + n, B, H, n, n + 3, 64)
    lb = d["log_beta"]
    rng = np.random.default_rng(n)
    bits = rng.integers(1, 1 << 23, n).astype(np.uint32) | np.uint32(0x80000000)
    lb[0, 0, :n] = np.where(np.arange(n) % 2 == 0, bits.view(np.float32),
                            np.float32(-1e-37))                 # subnormal and tiny normal
    lb[0, 1, :n] = (-rng.uniform(1e-44, 1e-35, n)).astype(np.float32)  # across the boundary
    lb[0, 1, 100:300] = lb[0, 1, 99]                            # equal keys by slot
    lb[1, :, :n] = (-rng.uniform(0.0, 1e-3, (H, n))).astype(np.float32)
    t = np.array([n + 5, (1 << 25) + 7], np.int32)              # row 1: d > 2^24
    for M in (n // 3, n - 1):
        _evict_and_check(d, t, M, f"subnormal/far n={n} M={M}")


def test_evict_float32_tiny_workload_steps():
    """The tiny workload: 16 decode steps of append + attention + eviction."""
    w = synth.WORKLOADS["tiny"]
    d = synth.host_cache(w)
    qs = synth.host_queries(w)
    kn, vn, lbn = synth.host_new_tokens(w)
    c = dev_cache(d)
    ref = oracle.Cache.from_arrays(d)
    for s in range(w.steps):
        say("tiny step", s)
        t = np.full(w.batch, w.ctx + s, np.int32)
        out, lse = kvb.kv_attn_decode(c, to_dev(qs[s]), to_dev(t), k_new=to_dev(kn[s]),
                                      v_new=to_dev(vn[s]), log_beta_new=to_dev(lbn[s]))
        n_ev = kvb.kv_evict_to_budget(c, to_dev(t), w.budget)
        torch.cuda.synchronize()
        oracle.append_tokens(ref, kn[s], vn[s], lbn[s], t)
        ref_out, ref_lse = oracle.decode_attention(ref.values("k"), ref.values("v"), ref.log_beta,
                                                   ref.pos, ref.length, qs[s].astype(np.float64), t)
        check_attention(to_host(out), to_host(lse), ref_out, ref_lse, f"tiny step {s}")
        ref, _, ref_n = oracle.evict_to_budget(ref, t, w.budget)
        check_layout(host_dict(c), ref, f"tiny step {s}")
        assert np.array_equal(to_host(n_ev), ref_n)


def test_evict_steady_state_shift():
    """Budget M with one token over: each step evicts one and shifts the rest down
    (the compaction's cross-workgroup staging path)."""
    B, H, D, M = 2, 2, 128, 1000
    d = _cache(21, B, H, M, M + 40, D)
    c = dev_cache(d)
    ref = oracle.Cache.from_arrays(d)
    rng = np.random.default_rng(5)
    for s in range(6):
        t = np.full(B, M + s, np.int32)
        kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        lbn = np.log(rng.uniform(0.5, 1.0, (B, H))).astype(np.float32)
        qn = synth.bf16_bits(rng.standard_normal((B, 4 * H, D)))
        kvb.kv_attn_decode(c, to_dev(qn), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                           log_beta_new=to_dev(lbn))
        kvb.kv_evict_to_budget(c, to_dev(t), M)
        torch.cuda.synchronize()
        oracle.append_tokens(ref, kn, vn, lbn, t)
        ref, _, _ = oracle.evict_to_budget(ref, t, M)
        check_layout(host_dict(c), ref, f"steady step {s}")


def test_evict_ties_and_special_keys_large_heads():
    """The chunked selection (heads too long for the LDS planner, 40,000 slots):
    all keys equal (evict by position), log beta = -inf every third slot, +0 / -0
    and a slot at the decode position, and a cluster of 20,000 keys that round to
    the same few float32 values but differ as doubles (lb_i = fl32(c / d_i)), the
    eviction threshold inside the cluster so the exact 64-bit pass and the slot
    search among exact ties both run."""
    B, H, n = 1, 4, 40000
    d = _cache(5, B, H, n, n + 3, 64)
    lb = d["log_beta"]
    t = np.array([n - 1], np.int32)                # pos n-1 sits at distance 0
    lb[0, 0, :n] = np.float32(0.0)                  # every key 0
    lb[0, 1, ::3] = -np.inf
    lb[0, 3, :n] = np.where(np.arange(n) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    lb[0, 3, 1000:30000] = np.float32(-0.001)
    dist = (t[0] - np.arange(n)).astype(np.float64)
    cl = np.arange(5000, 25000)
    c = -5.0
    lb[0, 2, cl] = (c / dist[cl]).astype(np.float32)
    keys = dist * lb[0, 2, :n].astype(np.float64)
    below = int(np.sum(keys < keys[cl].min()))
    kc = keys[cl]
    assert len(np.unique(kc.astype(np.float32))) < 40 < len(np.unique(kc))  # float32 ties
    for M in (1, 20000, 39999, n - below - 10000):
        _evict_and_check(d, t, M, f"large ties M={M}", max_evict=64)


def test_evict_large_head_bucket_in_one_slice():
    """Chunked selection where the threshold's bucket (3000 keys sharing their top
    11 bits, all in one 8192-slot slice) holds more members than a slice lists in
    LDS, so part of the list goes to the head's list directly; the threshold sits
    inside the bucket."""
    B, H, n = 1, 2, 40000
    d = _cache(9, B, H, n, n + 3, 128)
    lb = d["log_beta"]
    t = np.array([n], np.int32)
    dist = (t[0] - np.arange(n)).astype(np.float64)
    lb[0, :, :n] = np.float32(-1e-4)
    cl = np.arange(10000, 13000)
    for g in range(H):
        lb[0, g, cl] = (-1000.0 * (1.0 + 1e-4 * ((cl * (7 + g)) % 97)) / dist[cl]).astype(np.float32)
    keys = dist[cl] * lb[0, 0, cl].astype(np.float64)
    assert np.all(np.abs(keys) > 999) and np.all(np.abs(keys) < 1011)
    for M in (n - 1500, n - 2999, n - 1):
        _evict_and_check(d, t, M, f"bucket in one slice M={M}", max_evict=64)


def test_evict_dense_bucket_exact_fallback():
    """Chunked selection where more than 4096 keys (8000, spread over ~1000 float32
    values) share the threshold's 22-bit float32 bucket, so the selection finishes
    by exact passes over the head; the threshold sits inside that bucket."""
    B, H, n = 1, 2, 40000
    d = _cache(13, B, H, n, n + 3, 64)
    lb = d["log_beta"]
    t = np.array([n], np.int32)
    dist = (t[0] - np.arange(n)).astype(np.float64)
    lb[0, :, :n] = np.float32(-1e-4)                 # keys above -4: kept first
    cl = np.arange(15000, 23000)
    rng = np.random.default_rng(13)
    for g in range(H):
        kap = -1000.001 - 0.06 * rng.random(cl.size)   # inside one 1/16-wide bucket
        lb[0, g, cl] = (kap / dist[cl]).astype(np.float32)
    lb[0, :, :5000] = np.float32(-1.0)                # keys below the cluster: evicted first
    keys = dist[cl] * lb[0, 0, cl].astype(np.float64)
    k32 = np.unique(keys.astype(np.float32).view(np.uint32) >> 10)
    assert k32.size == 1, "the cluster shares its top 22 float32 bits"
    for M in (n - 5000 - 4000, n - 5000 - 7000, n - 5000 - 100):
        _evict_and_check(d, t, M, f"dense bucket M={M}", max_evict=64)


def test_evict_float32_and_d64():
    for dtype, D in (("f32", 64), ("bf16", 64), ("f32", 128)):
        d = _cache(31, 1, 2, 3000, 3001, D, dtype=dtype)
        _evict_and_check(d, np.array([3000], np.int32), 700, f"{dtype} D={D}")


@pytest.mark.parametrize("name", ["qwen3_8b_32k", "qwen3_32b_128k"])
def test_evict_full_size(name):
    """One full layer: append the decode token, evict every head to M.  The oracle's
    plan (from the downloaded retention arrays and positions) names the kept slots;
    every head's compacted rows must be exactly those rows, in order."""
    w = synth.WORKLOADS[name]
    say("evict full size", name)
    dc = synth.device_cache(w, layer=0)
    q, kn, vn, lbn = synth.device_queries(w, 0)
    t = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    c = kvb.KVCache.from_dict(dc)
    kvb.kv_attn_decode(c, q, t, k_new=kn, v_new=vn, log_beta_new=lbn)
    torch.cuda.synchronize()
    n = w.ctx + 1
    lbh = to_host(c.log_beta[:, :, :n])
    ph = to_host(c.pos[:, :, :n])
    keep, ref_ev = {}, {}
    for b in range(w.batch):
        for g in range(w.hkv):
            k, e = oracle.evict_plan(lbh[b, g], ph[b, g], n, w.ctx, w.budget)
            keep[(b, g)] = np.nonzero(k)[0]
            ref_ev[(b, g)] = e
    snap = snapshot_rows(c, keep)
    ev = torch.empty((w.batch, w.hkv, 64), dtype=torch.int32, device="cuda")
    n_ev = kvb.kv_evict_to_budget(c, t, w.budget, evicted_pos=ev)
    torch.cuda.synchronize()
    check_compacted(c, snap, name)
    assert (to_host(n_ev) == n - w.budget).all()
    evh = to_host(ev)
    for (b, g), e in ref_ev.items():
        assert np.array_equal(evh[b, g], e[:64]), f"evicted_pos ({b},{g})"
    del dc, c
    torch.cuda.empty_cache()


def test_erase_vs_oracle():
    rng = np.random.default_rng(9)
    for trial in range(6):
        B, H, n = 2, 3, int(rng.integers(1, 9000))
        d = _cache(40 + trial, B, H, n, n + 1, 128, retention=trial % 2 == 0)
        R = int(rng.integers(0, 40))
        ranges = np.zeros((B, R, 2), np.int32)
        nr = np.zeros(B, np.int32)
        for b in range(B):
            k = int(rng.integers(0, R + 1))
            edges = np.sort(rng.choice(n + 50, size=2 * k, replace=False)).astype(np.int32)
            ranges[b, :k] = edges.reshape(k, 2)
            nr[b] = k
        say("erase trial", trial, n, R)
        c = dev_cache(d)
        n_er = kvb.kv_erase_ranges(c, to_dev(ranges), to_dev(nr))
        torch.cuda.synchronize()
        ref, ref_n = oracle.erase_ranges(oracle.Cache.from_arrays(d),
                                         [ranges[b, :nr[b]] for b in range(B)])
        check_layout(host_dict(c), ref, f"erase {trial}")
        assert np.array_equal(to_host(n_er), ref_n)


def _erase_case(d, ranges, nr, what):
    B = d["len"].shape[0]
    c = dev_cache(d)
    n_er = kvb.kv_erase_ranges(c, to_dev(ranges), to_dev(nr))
    torch.cuda.synchronize()
    ref, ref_n = oracle.erase_ranges(oracle.Cache.from_arrays(d),
                                     [ranges[b, :nr[b]] for b in range(B)])
    check_layout(host_dict(c), ref, what)
    assert np.array_equal(to_host(n_er), ref_n), what


def test_erase_edge_cases():
    """Gapped positions (not equal to slots), ragged lengths per head, ranges that
    cover nothing, everything or a single slot, a small shift (most kept rows move by
    a few slots, so many sources lie in other groups' destinations), R = 0, and
    n_ranges below R with junk in the unused entries."""
    rng = np.random.default_rng(21)
    B, H, n, cap = 2, 3, 6000, 6100
    d = _cache(61, B, H, n, cap, 128, lens=[[6000, 17, 0], [1, 4321, 5999]])
    gaps = np.cumsum(rng.integers(1, 4, size=(B, H, cap)), axis=2).astype(np.int32)
    d["pos"] = gaps
    R = 6
    cases = {
        "nothing": [[(-100, -50)], [(10 ** 8, 10 ** 8 + 5)]],
        "everything": [[(0, 10 ** 8)], [(-5, 10 ** 8)]],
        "single slots": [[(int(gaps[0, 0, 5]), int(gaps[0, 0, 5]) + 1),
                          (int(gaps[0, 0, 100]), int(gaps[0, 0, 101]))],
                         [(int(gaps[1, 1, 0]), int(gaps[1, 1, 0]) + 1)]],
        "small shift": [[(0, int(gaps[0, 0, 7]))], [(int(gaps[1, 2, 3]), int(gaps[1, 2, 9]))]],
        "empty ranges": [[(5, 5), (9, 9)], [(7, 7)]],
        "many": [sorted_pairs(rng, 20000, 6), sorted_pairs(rng, 20000, 6)],
    }
    for name, per_b in cases.items():
        ranges = np.full((B, R, 2), 123456, np.int32)      # junk past n_ranges
        nr = np.zeros(B, np.int32)
        for b in range(B):
            for i, (s0, e0) in enumerate(per_b[b]):
                ranges[b, i] = (s0, e0)
            nr[b] = len(per_b[b])
        say("erase edge case", name)
        _erase_case(d, ranges, nr, name)
    say("erase R = 0")
    _erase_case(d, np.zeros((B, 0, 2), np.int32), np.zeros(B, np.int32), "R = 0")


def sorted_pairs(rng, hi, k):
    e = np.sort(rng.choice(hi, size=2 * k, replace=False))
    return [(int(e[2 * i]), int(e[2 * i + 1])) for i in range(k)]


def test_erase_many_ranges_chunked_path():
    """More ranges than the endpoint tables hold for this capacity: the per-chunk
    scan path."""
    rng = np.random.default_rng(23)
    B, H, n, cap = 2, 2, 3000, 3000
    d = _cache(63, B, H, n, cap, 128)
    R = 300
    ranges = np.zeros((B, R, 2), np.int32)
    nr = np.array([R, 170], np.int32)
    for b in range(B):
        ranges[b, :nr[b]] = np.array(sorted_pairs(rng, 3100, int(nr[b])), np.int32)
    say("erase chunked path", R)
    _erase_case(d, ranges, nr, "many ranges")


def test_memento_full_size():
    """1M-token cache laid out as thinking blocks + 200-token mementos: erase all
    completed blocks, append the decode token, attend with beta == 1, evict to M
    (a no-op here)."""
    w = synth.WORKLOADS["memento_1m"]
    blocks, ranges = synth.memento_layout(total=w.ctx, seed=w.seed)
    say("memento blocks", len(blocks), "ranges", ranges.shape)
    dc = synth.device_cache(w, layer=0)
    q, kn, vn, _ = synth.device_queries(w, 0)
    c = kvb.KVCache.from_dict(dc)
    ph = to_host(c.pos[:, :, :w.ctx])
    keep = {(0, g): np.nonzero(oracle.erase_plan(ph[0, g], w.ctx, ranges))[0]
            for g in range(w.hkv)}
    kept = 200 * (len(blocks) - 1) + blocks[-1][1]
    assert all(v.size == kept for v in keep.values())
    snap = snapshot_rows(c, keep)
    rg = torch.from_numpy(ranges[None].copy()).cuda()
    nr = torch.tensor([ranges.shape[0]], dtype=torch.int32, device="cuda")
    n_er = kvb.kv_erase_ranges(c, rg, nr)
    torch.cuda.synchronize()
    check_compacted(c, snap, "memento erase")
    assert (to_host(n_er) == w.ctx - kept).all()
    t = torch.full((1,), w.ctx, dtype=torch.int32, device="cuda")
    out, lse = kvb.kv_attn_decode(c, q, t, k_new=kn, v_new=vn)
    n_ev = kvb.kv_evict_to_budget(c, t, w.budget)
    torch.cuda.synchronize()
    assert to_host(n_ev).tolist() == [[0] * w.hkv]
    assert (to_host(c.length) == kept + 1).all()
    G = w.group
    oh, lh, qh = to_host(out), to_host(lse), to_host(q)
    knh, vnh = to_host(kn), to_host(vn)
    for g in (0, 5):
        s = snap[(0, g)]
        kk = np.concatenate([s["k"], knh[0, g][None]])[None, None]
        vv = np.concatenate([s["v"], vnh[0, g][None]])[None, None]
        pp = np.concatenate([s["pos"], [w.ctx]])[None, None]
        ro, rl = oracle.decode_attention(values(kk), values(vv), None, pp,
                                         np.array([[kept + 1]]),
                                         values(qh[:, g * G:(g + 1) * G]), np.array([w.ctx]))
        check_attention(oh[:, g * G:(g + 1) * G], lh[:, g * G:(g + 1) * G], ro, rl,
                        f"memento attention g={g}")
    del dc, c
    torch.cuda.empty_cache()


def test_steady_state_full_shape():
    """The 32K workload's layer shape at its budget: every head holds M = 4096
    tokens; three steps of append + attention + evict 1 + compact.  Every head's
    compacted rows against the oracle's plan; attention of sampled heads against the
    oracle."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    M = w.budget
    dc = synth.device_cache(w, layer=3, n=M, cap=M + 32)
    c = kvb.KVCache.from_dict(dc)
    G = w.group
    for s in range(3):
        say("steady step", s)
        q, kn, vn, lbn = synth.device_queries(w, 3, step=s)
        t = torch.full((w.batch,), M + s, dtype=torch.int32, device="cuda")
        kvb.kv_append(c, kn, vn, lbn, t)
        torch.cuda.synchronize()
        n = M + 1
        units = [(0, 0), (9, 5), (15, 7)]
        sub = {(b, g): {k: to_host(getattr(c, k)[b:b + 1, g:g + 1, :n])
                        for k in ("k", "v", "log_beta", "pos")} for (b, g) in units}
        out, lse = kvb.kv_attn_decode(c, q, t)
        lbh = to_host(c.log_beta[:, :, :n])
        ph = to_host(c.pos[:, :, :n])
        keep = {}
        for b in range(w.batch):
            for g in range(w.hkv):
                k, _ = oracle.evict_plan(lbh[b, g], ph[b, g], n, M + s, M)
                keep[(b, g)] = np.nonzero(k)[0]
        snap = snapshot_rows(c, keep)
        n_ev = kvb.kv_evict_to_budget(c, t, M)
        torch.cuda.synchronize()
        check_compacted(c, snap, f"steady {s}")
        assert (to_host(n_ev) == 1).all()
        oh, lh, qh = to_host(out), to_host(lse), to_host(q)
        for (b, g), d in sub.items():
            ro, rl = oracle.decode_attention(values(d["k"]), values(d["v"]), d["log_beta"],
                                             d["pos"], np.array([[n]], np.int32),
                                             values(qh[b:b + 1, g * G:(g + 1) * G]),
                                             np.array([M + s]))
            check_attention(oh[b:b + 1, g * G:(g + 1) * G], lh[b:b + 1, g * G:(g + 1) * G],
                            ro, rl, f"steady {s} ({b},{g})")
    del dc, c
    torch.cuda.empty_cache()
