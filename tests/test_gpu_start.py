"""Caches with a per-head first live slot (kvb_cache.start; a head's slots are a
ring): attention, append, eviction (toward either end of the head), erasure and
the latent update on the GPU, checked on the live rows against the oracle, which
knows only the logical (slot 0 based) layout."""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import (check_attention, check_layout, oracle_attention, say, to_dev, to_host,
                      values)

pytestmark = pytest.mark.gpu


def _dense(seed, B, Hkv, n, cap, D, dtype="bf16", retention=True, lens=None):
    w = synth.Workload("t", batch=B, hq=Hkv, hkv=Hkv, head_dim=D, dtype=dtype, ctx=n,
                       budget=0, layers=1, seed=seed, retention=retention)
    d = synth.host_cache(w, n=n, cap=cap)
    if lens is not None:
        d["len"] = np.asarray(lens, np.int32).reshape(B, Hkv)
    return d


def _ring(s, n, cap):
    return (s + np.arange(n)) % cap


def _placed(d, starts, cap, seed):
    """Device cache holding head (b, g)'s live rows at slots starts[b, g] + i (mod
    cap) of a cap-slot buffer; every other slot holds large garbage values."""
    B, H = d["len"].shape
    D = d["k"].shape[-1]
    rng = np.random.default_rng(seed)
    ph = {}
    for name in ("k", "v"):
        g = rng.standard_normal((B, H, cap, D)) * 1e3
        ph[name] = synth.bf16_bits(g) if d[name].dtype == np.uint16 else g.astype(np.float32)
    ph["pos"] = rng.integers(-(1 << 30), 1 << 30, (B, H, cap)).astype(np.int32)
    ph["log_beta"] = None if d["log_beta"] is None else \
        (-rng.uniform(0, 50, (B, H, cap))).astype(np.float32)
    for b in range(B):
        for g in range(H):
            s, n = int(starts[b, g]), int(d["len"][b, g])
            assert 0 <= s < cap and n <= cap
            for name in ("k", "v", "pos", "log_beta"):
                if ph[name] is not None:
                    ph[name][b, g, _ring(s, n, cap)] = d[name][b, g, :n]
    return kvb.KVCache(to_dev(ph["k"]), to_dev(ph["v"]), to_dev(ph["log_beta"]),
                       to_dev(ph["pos"]), to_dev(d["len"]),
                       start=to_dev(np.asarray(starts, np.int32)))


def _logical(c: kvb.KVCache):
    """Host copy of the live rows of every head moved to slot 0 (cap slots wide)."""
    k, v, pos = to_host(c.k), to_host(c.v), to_host(c.pos)
    lb = to_host(c.log_beta)
    ln, st = to_host(c.length), to_host(c.start)
    out = {"k": np.zeros_like(k), "v": np.zeros_like(v), "pos": np.zeros_like(pos),
           "log_beta": None if lb is None else np.zeros_like(lb), "len": ln}
    B, H = ln.shape
    for b in range(B):
        for g in range(H):
            s, n = int(st[b, g]), int(ln[b, g])
            assert 0 <= s < c.cap and n <= c.cap, f"({b},{g}) start {s} len {n} cap {c.cap}"
            for name, src in (("k", k), ("v", v), ("pos", pos), ("log_beta", lb)):
                if src is not None:
                    out[name][b, g, :n] = src[b, g, _ring(s, n, c.cap)]
    return out


def _expected_start(d, ref_ev, s0, cap):
    """First live slot after eviction by the rule: toward whichever end of the head
    moves fewer kept rows (toward its last slot the first slot advances by the
    evicted count, around the ring)."""
    B, H = d["len"].shape
    ns = np.array(s0, np.int64).copy()
    for b in range(B):
        for g in range(H):
            n = int(d["len"][b, g])
            ev = np.asarray(ref_ev[b][g])
            if len(ev) == 0:
                continue
            slots = np.searchsorted(d["pos"][b, g, :n], ev)
            nev, kept = len(ev), n - len(ev)
            fwd = kept - int(slots.min())
            bwd = int(slots.max()) + 1 - nev
            if bwd < fwd:
                ns[b, g] = (s0[b, g] + nev) % cap
    return ns


@pytest.mark.parametrize("D,dtype,Hq,Hkv", [(128, "bf16", 8, 2), (64, "bf16", 8, 2),
                                            (64, "f32", 4, 2), (128, "bf16", 6, 2)])
@pytest.mark.parametrize("append", [False, True])
def test_start_attention(D, dtype, Hq, Hkv, append):
    """Attention (and the decode-token append) over heads that start at odd slots."""
    B, cap = 2, 1500
    lens = np.array([[700, 1], [0, 1300]], np.int32)[:, :Hkv]
    d = _dense(5 + D, B, Hkv, 1300, 1300 + 1, D, dtype, lens=lens)
    rng = np.random.default_rng(D)
    starts = np.array([[3, 1498], [77, 1400]], np.int32)[:, :Hkv]  # (1, 1) wraps
    say("start attention", D, dtype, Hq, Hkv, append, starts.tolist())
    c = _placed(d, starts, cap, 11)
    q = synth.bf16_bits(rng.standard_normal((B, Hq, D))) if dtype == "bf16" else \
        rng.standard_normal((B, Hq, D)).astype(np.float32)
    t = np.array([1400, 1310], np.int32)
    ref = oracle.Cache.from_arrays(d)
    if append:
        kn = q[:, :Hkv] * 1
        vn = q[:, Hkv:2 * Hkv] * 1
        lbn = np.log(rng.uniform(0.5, 1.0, (B, Hkv))).astype(np.float32)
        out, lse = kvb.kv_attn_decode(c, to_dev(q), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                                      log_beta_new=to_dev(lbn))
        oracle.append_tokens(ref, kn, vn, lbn, t)
    else:
        out, lse = kvb.kv_attn_decode(c, to_dev(q), to_dev(t))
    torch.cuda.synchronize()
    rd = {"k": ref.k, "v": ref.v, "log_beta": ref.log_beta, "pos": ref.pos, "len": ref.length}
    ro, rl = oracle_attention(rd, q, t)
    check_attention(to_host(out), to_host(lse), ro, rl, "start attention")
    assert np.array_equal(to_host(c.start), starts), "attention must not move a head"
    check_layout(_logical(c), ref, "start attention layout")


def test_start_evict_directions():
    """One batch whose heads compact toward their first or their last slot, some of
    them wrapped around the end of their slots; budget one below the length."""
    B, H, n, cap, D = 1, 7, 600, 640, 128
    d = _dense(21, B, H, n, n, D)
    lb = d["log_beta"]
    lb[0, :, :] = np.float32(-1e-4)
    lb[0, 0, 5] = -5.0     # early eviction: toward the last slot
    lb[0, 1, 5] = -5.0     # early eviction in a wrapped head
    lb[0, 2, 590] = -5.0   # late eviction: toward the first slot
    lb[0, 3, 300] = -5.0   # middle
    lb[0, 4, 5] = -5.0     # early eviction, head at slot 0
    lb[0, 5, 0] = -5.0     # the first slot: nothing moves
    lb[0, 6, 2] = -5.0     # the first slot moves past the end of the slots to 0
    starts = np.array([[10, cap - 100, 17, 3, 0, 25, cap - 1]], np.int32)
    t = np.array([n + 10], np.int32)
    c = _placed(d, starts, cap, 3)
    kvb.kv_evict_to_budget(c, to_dev(t), n - 1)
    torch.cuda.synchronize()
    ref, ref_ev, _ = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, n - 1)
    check_layout(_logical(c), ref, "directions")
    ns = to_host(c.start)
    want = _expected_start(d, ref_ev, starts, cap)
    say("starts", starts.tolist(), "->", ns.tolist())
    assert np.array_equal(ns, want), f"{ns} vs {want}"
    assert list(ns[0]) == [11, cap - 99, 17, 3, 1, 26, 0]


@pytest.mark.parametrize("n,M", [(513, 256), (4097, 4096), (5000, 64), (3000, 2999), (9000, 1)])
@pytest.mark.parametrize("retention", [True, False])
def test_start_evict_bulk(n, M, retention):
    """Bulk eviction with random starts (most heads wrap around their slots)."""
    B, H = 2, 3
    cap = n + 40
    d = _dense(n + M, B, H, n, n, 128, retention=retention)
    rng = np.random.default_rng(n)
    starts = rng.integers(0, cap, (B, H)).astype(np.int32)
    starts[0, 0] = cap - n
    starts[1, 2] = 0
    t = np.array([n + 2, n + 9], np.int32)
    say("start bulk", n, M, retention, starts.tolist())
    c = _placed(d, starts, cap, 5)
    me = n
    ev = torch.full((B, H, me), -7, dtype=torch.int32, device="cuda")
    n_ev = kvb.kv_evict_to_budget(c, to_dev(t), M, evicted_pos=ev)
    torch.cuda.synchronize()
    ref, ref_ev, ref_n = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    check_layout(_logical(c), ref, f"bulk n={n} M={M}")
    assert np.array_equal(to_host(n_ev), ref_n)
    evh = to_host(ev)
    for b in range(B):
        for g in range(H):
            k = int(ref_n[b, g])
            assert np.array_equal(evh[b, g, :k], ref_ev[b][g][:k])
    assert np.array_equal(to_host(c.start), _expected_start(d, ref_ev, starts, cap))


def test_start_evict_large_head():
    """A head too long for the LDS planner (chunked selection): compacted toward its
    first slot, start kept; one head wraps."""
    B, H, n, M = 1, 2, 40000, 5000
    cap = n + 100
    d = _dense(77, B, H, n, n, 128)
    starts = np.array([[100, cap - 37]], np.int32)
    t = np.array([n], np.int32)
    c = _placed(d, starts, cap, 8)
    kvb.kv_evict_to_budget(c, to_dev(t), M)
    torch.cuda.synchronize()
    ref, _, _ = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    check_layout(_logical(c), ref, "large head")
    assert np.array_equal(to_host(c.start), starts)


def test_start_erase():
    """Range erasure keeps each head's start and compacts toward it."""
    rng = np.random.default_rng(12)
    B, H, n, cap = 2, 3, 5000, 5300
    d = _dense(31, B, H, n, n, 128)
    starts = rng.integers(0, cap, (B, H)).astype(np.int32)
    R = 30
    ranges = np.zeros((B, R, 2), np.int32)
    nr = np.zeros(B, np.int32)
    for b in range(B):
        k = int(rng.integers(1, R + 1))
        edges = np.sort(rng.choice(n + 50, size=2 * k, replace=False)).astype(np.int32)
        ranges[b, :k] = edges.reshape(k, 2)
        nr[b] = k
    c = _placed(d, starts, cap, 9)
    n_er = kvb.kv_erase_ranges(c, to_dev(ranges), to_dev(nr))
    torch.cuda.synchronize()
    ref, ref_n = oracle.erase_ranges(oracle.Cache.from_arrays(d),
                                     [ranges[b, :nr[b]] for b in range(B)])
    check_layout(_logical(c), ref, "erase with starts")
    assert np.array_equal(to_host(n_er), ref_n)
    assert np.array_equal(to_host(c.start), starts)


@pytest.mark.parametrize("one", [False, True])
def test_start_steady_loop(one):
    """Decode steps at budget M (append, attend, evict one) with and without a start
    array, 4 spare slots: outputs bit-identical, layouts equal to the oracle, and
    heads wrap around the end of their slots.  Eviction by kv_evict_to_budget, or
    by kv_evict_one."""
    B, H, Hq, D, M = 2, 2, 8, 128, 300
    cap = M + 4
    d = _dense(41, B, H, M, cap, D)
    plain = kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]),
                        to_dev(d["pos"]), to_dev(d["len"]))
    st = kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]),
                     to_dev(d["pos"]), to_dev(d["len"]),
                     start=torch.zeros((B, H), dtype=torch.int32, device="cuda"))
    ref = oracle.Cache.from_arrays(d)
    rng = np.random.default_rng(2)
    seen, wrapped = set(), False
    for s in range(24):
        t = np.full(B, M + s, np.int32)
        kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        lbn = np.log(rng.uniform(0.3, 1.0, (B, H))).astype(np.float32)
        q = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
        outs = []
        for c in (plain, st):
            o, l = kvb.kv_attn_decode(c, to_dev(q), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                                      log_beta_new=to_dev(lbn))
            if one:
                ne = kvb.kv_evict_one(c, to_dev(t), M)
                assert bool((ne == 1).all())
            else:
                kvb.kv_evict_to_budget(c, to_dev(t), M)
            outs.append((o, l))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), s
        oracle.append_tokens(ref, kn, vn, lbn, t)
        ref, _, _ = oracle.evict_to_budget(ref, t, M)
        check_layout(_logical(st), ref, f"steady step {s}")
        sv = to_host(st.start)
        seen.update(int(x) for x in sv.ravel())
        wrapped = wrapped or bool((sv + to_host(st.length) > cap).any())
    say("starts seen", sorted(seen))
    assert len(seen) > 1 and wrapped


def test_start_latent_absorb():
    """The latent memory update reads the evicted rows where the head starts."""
    B, H, n, M, D = 1, 2, 3000, 1000, 128
    cap = n + 50
    d = _dense(51, B, H, n, n, D)
    starts = np.array([[50, cap - 13]], np.int32)
    t = np.array([n + 1], np.int32)
    res = []
    for placed in (False, True):
        if placed:
            c = _placed(d, starts, cap, 4)
        else:
            c = kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]),
                            to_dev(d["pos"]), to_dev(d["len"]))
        ws = torch.empty(kvb.kv_evict_workspace(c, M), dtype=torch.uint8, device="cuda")
        kvb.kv_evict_plan(c, to_dev(t), M, ws=ws)
        mem_M = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
        mem_b = torch.zeros((B, H, D), dtype=torch.float32, device="cuda")
        kvb.kv_latent_absorb(c, M, ws, 0.999, mem_M, mem_b)
        torch.cuda.synchronize()
        res.append((to_host(mem_M), to_host(mem_b)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    ev = []
    _, ref_ev, _ = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    for g in range(H):
        slots = np.searchsorted(d["pos"][0, g, :n], ref_ev[0][g])
        Mref, bref = oracle.latent_absorb(np.zeros((D, D)), np.zeros(D),
                                          values(d["k"][0, g, slots]), values(d["v"][0, g, slots]),
                                          0.999)
        err = np.max(np.abs(res[1][0][0, g] - Mref)) / np.max(np.abs(Mref))
        ev.append(err)
        assert err < 1e-3, (g, err)
    say("latent rel err", ev)


def test_start_fused_entry_falls_back():
    """kv_attn_decode_compact on ring heads takes the unfused path: attention, then
    the planned compaction (toward either end), as separate calls would."""
    B, H, Hq, n, M, D = 1, 2, 8, 2000, 700, 128
    cap = n + 64
    d = _dense(61, B, H, n, n, D)
    starts = np.array([[9, cap - 500]], np.int32)
    rng = np.random.default_rng(6)
    q = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
    t = np.array([n + 4], np.int32)
    c = _placed(d, starts, cap, 2)
    ws_e = torch.empty(kvb.kv_evict_workspace(c, M), dtype=torch.uint8, device="cuda")
    kvb.kv_evict_plan(c, to_dev(t), M, ws=ws_e)
    out, lse = kvb.kv_attn_decode_compact(c, to_dev(q), to_dev(t), M, ws_e)
    torch.cuda.synchronize()
    ro, rl = oracle_attention(d, q, t)
    check_attention(to_host(out), to_host(lse), ro, rl, "fused entry on ring heads")
    ref, ref_ev, _ = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    check_layout(_logical(c), ref, "fused entry layout")
    assert np.array_equal(to_host(c.start), _expected_start(d, ref_ev, starts, cap))


def _copy_cache(c: kvb.KVCache) -> kvb.KVCache:
    cl = (lambda x: None if x is None else x.clone())
    return kvb.KVCache(cl(c.k), cl(c.v), cl(c.log_beta), cl(c.pos), cl(c.length),
                       start=cl(c.start))


def _same_cache(c1: kvb.KVCache, c2: kvb.KVCache, what):
    """Bit-equal lengths, starts and live rows (slot by slot)."""
    assert torch.equal(c1.length, c2.length), f"{what} len"
    if c1.start is not None:
        assert torch.equal(c1.start, c2.start), f"{what} start"
    ln = to_host(c1.length)
    st = to_host(c1.start) if c1.start is not None else np.zeros_like(ln)
    cap = c1.k.shape[2]
    arrs = [(to_host(getattr(c1, nm)), to_host(getattr(c2, nm)), nm)
            for nm in ("k", "v", "pos", "log_beta") if getattr(c1, nm) is not None]
    for b in range(ln.shape[0]):
        for g in range(ln.shape[1]):
            sl = _ring(int(st[b, g]), int(ln[b, g]), cap)
            for x1, x2, nm in arrs:
                assert np.array_equal(x1[b, g, sl], x2[b, g, sl]), f"{what} ({b},{g}) {nm}"


@pytest.mark.parametrize("ring", [True, False])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_evict_one_equals_evict_to_budget(ring, dtype, D):
    """kv_evict_one on heads one token over M: the same evicted position, layout,
    len and start as kv_evict_to_budget (evicted slot at the first / last slot, in
    the middle, at the tie e = n - 1 - e, equal keys resolved by slot, log beta =
    -inf), heads at or below M untouched, heads further over flagged and untouched;
    the logical layout also against the oracle."""
    B, H, M = 2, 6, 300
    n = M + 1
    cap = n + 20
    d = _dense(11 + D, B, H, n, cap, D, dtype=dtype)
    lb = d["log_beta"]
    lb[0, 0, :n] = -0.5
    lb[0, 0, 0] = -60.0                                      # lowest key at slot 0
    lb[0, 1, :n] = -0.01
    lb[0, 1, n - 1] = -np.inf                                # at the last slot
    lb[0, 2, :n] = 0.0                                       # every key 0: slot 0 goes
    lb[0, 3, :n] = -0.01
    lb[0, 3, 150] = -np.inf                                  # e = 150 = n - 1 - e
    lb[0, 4, :n] = -0.01
    lb[0, 4, 149] = -np.inf                                  # just below the middle
    lb[1, 0, :n] = -0.01
    lb[1, 0, 151] = -np.inf                                  # just above the middle
    d["len"][1, 1] = M                                       # at budget: untouched
    d["len"][1, 2] = M - 7
    d["len"][1, 3] = M + 3                                   # further over: flagged
    t = np.array([n + 2, n + 9], np.int32)
    rng = np.random.default_rng(D)
    starts = np.zeros((B, H), np.int64)
    if ring:
        starts = rng.integers(0, cap, (B, H))
        starts[0, 5] = cap - 1                               # the ring wraps at once
    c1 = _placed(d, starts, cap, 3)
    if not ring:
        c1 = kvb.KVCache(c1.k, c1.v, c1.log_beta, c1.pos, c1.length)
    c2 = _copy_cache(c1)
    say("evict_one", ring, dtype, D)
    ev1 = torch.full((B, H, 2), -7, dtype=torch.int32, device="cuda")
    n1 = kvb.kv_evict_one(c1, to_dev(t), M, evicted_pos=ev1)
    torch.cuda.synchronize()
    n1h = to_host(n1)
    assert n1h[1, 3] == -3 and n1h[1, 1] == 0 and n1h[1, 2] == 0
    assert int(to_host(c1.length)[1, 3]) == M + 3, "flagged head untouched"
    # the general path on the copy, with the flagged head brought to M + 1 first
    # in neither: compare every other head
    ev2 = torch.full((B, H, 2), -7, dtype=torch.int32, device="cuda")
    keep13 = c2.length[1, 3].item()
    c2.length[1, 3] = M
    n2 = kvb.kv_evict_to_budget(c2, to_dev(t), M, evicted_pos=ev2)
    torch.cuda.synchronize()
    c2.length[1, 3] = keep13
    n2h = to_host(n2)
    n2h[1, 3] = -3
    assert np.array_equal(n1h, n2h), "n_evicted"
    e1, e2 = to_host(ev1), to_host(ev2)
    for b in range(B):
        for g in range(H):
            if n1h[b, g] == 1:
                assert e1[b, g, 0] == e2[b, g, 0], f"evicted pos ({b},{g})"
    if ring:
        st1, st2 = to_host(c1.start), to_host(c2.start)
        assert np.array_equal(np.delete(st1.ravel(), 9), np.delete(st2.ravel(), 9))
    # the flagged head's rows were never touched in either; compare the others
    c2.length[1, 3] = c1.length[1, 3]
    if ring:
        c2.start[1, 3] = c1.start[1, 3]
    _same_cache(c1, c2, f"evict_one ring={ring} {dtype} D={D}")
    # against the oracle (logical layout; the flagged head excluded)
    dd = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    dd["len"][1, 3] = M
    ref, _, _ = oracle.evict_to_budget(oracle.Cache.from_arrays(dd), t, M)
    got = _logical(c1) if ring else {"k": to_host(c1.k), "v": to_host(c1.v),
                                     "log_beta": to_host(c1.log_beta), "pos": to_host(c1.pos),
                                     "len": to_host(c1.length)}
    got["len"] = got["len"].copy()
    got["len"][1, 3] = M
    check_layout(got, ref, f"evict_one oracle ring={ring}")
