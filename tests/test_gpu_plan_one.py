"""The steady state's eviction selected by the attention (kv_attn_decode_plan_one)
and applied by kv_evict_one_apply: the attention bit for bit as kv_attn_decode,
the eviction bit for bit as kv_evict_one (same evicted position, direction, layout,
len and start), and the layouts of a decode loop against the oracle."""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import check_attention, check_layout, oracle_attention, say, to_dev, to_host
from test_gpu_start import _copy_cache, _dense, _logical, _placed, _same_cache

pytestmark = pytest.mark.gpu


def _special_keys(d, n, M):
    """Heads whose lowest key sits at slot 0, at the last cached slot, in the middle
    and on either side of it, with every key equal (slot 0 goes), log beta = -inf;
    one head at M, one below, one further over."""
    lb = d["log_beta"]
    if lb is None:
        return
    lb[0, 0, :n] = -0.5
    lb[0, 0, 0] = -60.0
    lb[0, 1, :n] = -0.01
    lb[0, 1, n - 1] = -np.inf
    lb[0, 2, :n] = 0.0
    lb[0, 3, :n] = -0.01
    lb[0, 3, n // 2] = -np.inf
    lb[0, 4, :n] = -0.01
    lb[0, 4, n // 2 - 1] = -np.inf
    lb[1, 0, :n] = -0.01
    lb[1, 0, n // 2 + 1] = -np.inf


@pytest.mark.parametrize("dtype,D,Hq", [("bf16", 128, 24), ("bf16", 128, 48), ("bf16", 64, 12),
                                        ("f32", 64, 12)])
@pytest.mark.parametrize("append", [True, False])
@pytest.mark.parametrize("ring", [True, False])
@pytest.mark.parametrize("P", [0, 1, 7, 64])
def test_plan_one_equals_attention_and_evict_one(dtype, D, Hq, append, ring, P):
    """Against kv_attn_decode + kv_evict_one on a copy of the same cache: out and lse
    bit for bit, n_evicted, evicted positions, len, start and the live rows bit for
    bit; heads at or under M untouched, a head further over flagged and untouched."""
    B, H, M = 2, 6, 300
    n = M if append else M + 1          # cached slots before the call
    cap = M + 24
    d = _dense(7 + D + Hq, B, H, n, cap, D, dtype=dtype)
    _special_keys(d, n, M)
    d["len"][1, 1] = M - (0 if not append else 1)   # at M after the call
    d["len"][1, 2] = M - 9
    d["len"][1, 3] = n + 2                          # further over after the call
    t = np.array([n + 3, n + 11], np.int32)
    rng = np.random.default_rng(D + Hq)
    starts = np.zeros((B, H), np.int64)
    if ring:
        starts = rng.integers(0, cap, (B, H))
        starts[0, 5] = cap - 1
    c1 = _placed(d, starts, cap, 5)
    if not ring:
        c1 = kvb.KVCache(c1.k, c1.v, c1.log_beta, c1.pos, c1.length)
    c2 = _copy_cache(c1)
    q = rng.standard_normal((B, Hq, D))
    q = synth.bf16_bits(q) if dtype == "bf16" else q.astype(np.float32)
    kn = vn = lbn = None
    if append:
        kn = rng.standard_normal((B, H, D))
        vn = rng.standard_normal((B, H, D))
        kn, vn = ((synth.bf16_bits(x) if dtype == "bf16" else x.astype(np.float32))
                  for x in (kn, vn))
        lbn = np.log(rng.uniform(0.2, 1.0, (B, H))).astype(np.float32)
    say("plan_one", dtype, D, Hq, "append", append, "ring", ring, "P", P)
    ws_e = torch.empty(kvb.kv_evict_one_workspace(c1, P), dtype=torch.uint8, device="cuda")
    o1, l1 = kvb.kv_attn_decode_plan_one(c1, to_dev(q), to_dev(t), ws_e, k_new=to_dev(kn),
                                         v_new=to_dev(vn), log_beta_new=to_dev(lbn),
                                         num_splits=P)
    ev1 = torch.full((B, H, 2), -7, dtype=torch.int32, device="cuda")
    n1 = kvb.kv_evict_one_apply(c1, to_dev(t), M, ws_e, evicted_pos=ev1)
    o2, l2 = kvb.kv_attn_decode(c2, to_dev(q), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                                log_beta_new=to_dev(lbn), num_splits=P)
    ev2 = torch.full((B, H, 2), -7, dtype=torch.int32, device="cuda")
    n2 = kvb.kv_evict_one(c2, to_dev(t), M, evicted_pos=ev2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "attention bit for bit"
    assert torch.equal(n1, n2), "n_evicted"
    n1h = to_host(n1)
    assert n1h[1, 3] == -3 and n1h[1, 1] == 0 and n1h[1, 2] == 0
    e1, e2 = to_host(ev1), to_host(ev2)
    assert np.array_equal(e1[n1h == 1][:, 0], e2[n1h == 1][:, 0]), "evicted positions"
    assert np.all(e1[n1h != 1] == -7), "no position for heads not evicted"
    _same_cache(c1, c2, f"plan_one {dtype} D={D} append={append} ring={ring} P={P}")
    # the attention against the oracle on the cache as it was before the call
    if append:
        dd = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
        ref = oracle.Cache.from_arrays(dd)
        oracle.append_tokens(ref, kn, vn, lbn, t)
        dd = {"k": ref.k, "v": ref.v, "log_beta": ref.log_beta, "pos": ref.pos,
              "len": ref.length}
    else:
        dd = d
    ro, rl = oracle_attention(dd, q, t)
    check_attention(to_host(o1), to_host(l1), ro, rl, "plan_one attention")


def test_plan_one_long_shift_chunks():
    """Heads of 4097 slots evicting near the middle: the shift runs in many chunks
    per head, each boundary row staged; the layout against kv_evict_one and the
    oracle."""
    B, H, Hq, D, M = 2, 4, 16, 128, 4096
    n = M
    cap = M + 32
    d = _dense(91, B, H, n, cap, D)
    lb = d["log_beta"]
    lb[:, :, :n] = -0.001
    for i, e in enumerate([0, 1, 63, 64, 65, 2047, 2048, 2049]):
        lb[i // H, i % H, e] = -np.inf
    rng = np.random.default_rng(3)
    starts = rng.integers(0, cap, (B, H))
    c1 = _placed(d, starts, cap, 8)
    c2 = _copy_cache(c1)
    q = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
    kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
    vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
    lbn = np.full((B, H), -0.001, np.float32)
    t = np.array([n + 1, n + 5], np.int32)
    ws_e = torch.empty(kvb.kv_evict_one_workspace(c1, 32), dtype=torch.uint8, device="cuda")
    kvb.kv_attn_decode_plan_one(c1, to_dev(q), to_dev(t), ws_e, k_new=to_dev(kn),
                                v_new=to_dev(vn), log_beta_new=to_dev(lbn), num_splits=32)
    n1 = kvb.kv_evict_one_apply(c1, to_dev(t), M, ws_e)
    kvb.kv_attn_decode(c2, to_dev(q), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                       log_beta_new=to_dev(lbn), num_splits=32)
    kvb.kv_evict_one(c2, to_dev(t), M)
    torch.cuda.synchronize()
    assert bool((n1 == 1).all())
    _same_cache(c1, c2, "long shift")
    ref = oracle.Cache.from_arrays(d)
    oracle.append_tokens(ref, kn, vn, lbn, t)
    ref, _, _ = oracle.evict_to_budget(ref, t, M)
    check_layout(_logical(c1), ref, "long shift vs oracle")


@pytest.mark.parametrize("ring", [True, False])
def test_plan_one_steady_loop(ring):
    """Decode steps at budget M with the attention and its planned eviction: each
    step's output within 2e-3 of the oracle's (append, attend, evict one) and the
    layout equal to the oracle's after every step; the apply runs on a second
    stream after an event, as a serving loop would run it."""
    B, H, Hq, D, M = 2, 2, 8, 128, 300
    cap = M + 4
    d = _dense(43, B, H, M, cap, D)
    c = kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]), to_dev(d["pos"]),
                    to_dev(d["len"]),
                    start=torch.zeros((B, H), dtype=torch.int32, device="cuda") if ring else None)
    ref = oracle.Cache.from_arrays(d)
    rng = np.random.default_rng(4)
    side = torch.cuda.Stream()
    ws_e = torch.empty(kvb.kv_evict_one_workspace(c, 0), dtype=torch.uint8, device="cuda")
    for s in range(20):
        t = np.full(B, M + s, np.int32)
        kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        lbn = np.log(rng.uniform(0.3, 1.0, (B, H))).astype(np.float32)
        q = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
        td = to_dev(t)
        o, l = kvb.kv_attn_decode_plan_one(c, to_dev(q), td, ws_e, k_new=to_dev(kn),
                                           v_new=to_dev(vn), log_beta_new=to_dev(lbn))
        done = torch.cuda.Event()
        done.record()
        side.wait_event(done)
        ne = kvb.kv_evict_one_apply(c, td, M, ws_e, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert bool((ne == 1).all()), s
        oracle.append_tokens(ref, kn, vn, lbn, t)
        ro, rl = oracle_attention({"k": ref.k, "v": ref.v, "log_beta": ref.log_beta,
                                   "pos": ref.pos, "len": ref.length}, q, t)
        check_attention(to_host(o), to_host(l), ro, rl, f"step {s}")
        ref, _, _ = oracle.evict_to_budget(ref, t, M)
        got = _logical(c) if ring else {"k": to_host(c.k), "v": to_host(c.v),
                                        "log_beta": to_host(c.log_beta), "pos": to_host(c.pos),
                                        "len": to_host(c.length)}
        check_layout(got, ref, f"steady plan_one step {s}")


def test_plan_one_full_shape_steps():
    """The steady state at the 32K workload's model shape (batch 16, 32 query / 8 KV
    heads, D = 128, M = 4096, ring heads): three steps against kv_attn_decode +
    kv_evict_one on a copy, attention and every head's layout bit for bit."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    M = w.budget
    dc = synth.device_cache(w, 0, n=M, cap=M + 32)
    B, H = w.batch, w.hkv
    dc["start"] = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    c1 = kvb.KVCache.from_dict(dc)
    c2 = _copy_cache(c1)
    q, kn, vn, lbn = synth.device_queries(w, 0)
    ws_e = torch.empty(kvb.kv_evict_one_workspace(c1, 32), dtype=torch.uint8, device="cuda")
    for s in range(3):
        t = torch.full((B,), M + s, dtype=torch.int32, device="cuda")
        say("full shape step", s)
        o1, l1 = kvb.kv_attn_decode_plan_one(c1, q, t, ws_e, k_new=kn, v_new=vn,
                                             log_beta_new=lbn, num_splits=32)
        n1 = kvb.kv_evict_one_apply(c1, t, M, ws_e)
        o2, l2 = kvb.kv_attn_decode(c2, q, t, k_new=kn, v_new=vn, log_beta_new=lbn,
                                    num_splits=32)
        n2 = kvb.kv_evict_one(c2, t, M)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), s
        assert bool((n1 == 1).all()) and torch.equal(n1, n2), s
        _same_cache(c1, c2, f"full shape step {s}")


def _by_position(c: kvb.KVCache):
    """Host copy of every head's live rows sorted by position (slot 0 based), for
    caches whose slots are not in position order (fill)."""
    got = _logical(c) if c.start is not None else {
        "k": to_host(c.k), "v": to_host(c.v), "log_beta": to_host(c.log_beta),
        "pos": to_host(c.pos), "len": to_host(c.length)}
    out = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in got.items()}
    B, H = out["len"].shape
    for b in range(B):
        for g in range(H):
            n = int(out["len"][b, g])
            order = np.argsort(got["pos"][b, g, :n], kind="stable")
            assert len(np.unique(got["pos"][b, g, :n])) == n, f"({b},{g}) positions repeat"
            for name in ("k", "v", "pos", "log_beta"):
                if out[name] is not None:
                    out[name][b, g, :n] = got[name][b, g, :n][order]
    return out


@pytest.mark.parametrize("dtype,D,Hq", [("bf16", 128, 24), ("bf16", 128, 48), ("bf16", 64, 12),
                                        ("f32", 64, 12)])
@pytest.mark.parametrize("ring", [True, False])
@pytest.mark.parametrize("append", [True, False])
@pytest.mark.parametrize("P", [0, 7, 100])
def test_evict_one_fill_equals_evict_one(dtype, D, Hq, ring, append, P):
    """kv_attn_decode_evict_one: the decode token (or, without one, the last live row)
    takes the evicted slot.  Against kv_attn_decode + kv_evict_one on a copy: out and
    lse bit for bit, n_evicted, the evicted positions and len equal, start unchanged,
    and the live rows equal as a set (bit for bit, sorted by position); 100 splits
    take the merge for many splits and the separate eviction kernel."""
    B, H, M = 2, 6, 300
    n = M if append else M + 1          # cached slots before the call
    cap = M + 24
    # rows (distinct positions) for the longest head, the others cut to n
    d = _dense(17 + D + Hq, B, H, n + 3, cap, D, dtype=dtype)
    d["len"][:] = n
    _special_keys(d, n, M)
    d["len"][1, 1] = M - (1 if append else 0)        # at M after the call
    d["len"][1, 2] = M - 9
    d["len"][1, 3] = n + 2                           # further over after the call
    t = np.array([n + 3 + 3, n + 11], np.int32)
    rng = np.random.default_rng(D + Hq + 1)
    starts = rng.integers(0, cap, (B, H)) if ring else np.zeros((B, H), np.int64)
    c1 = _placed(d, starts, cap, 5)
    if not ring:
        c1 = kvb.KVCache(c1.k, c1.v, c1.log_beta, c1.pos, c1.length)
    c2 = _copy_cache(c1)
    q = rng.standard_normal((B, Hq, D))
    q = synth.bf16_bits(q) if dtype == "bf16" else q.astype(np.float32)
    kn = vn = lbn = None
    if append:
        kn = rng.standard_normal((B, H, D))
        vn = rng.standard_normal((B, H, D))
        kn, vn = ((synth.bf16_bits(x) if dtype == "bf16" else x.astype(np.float32))
                  for x in (kn, vn))
        lbn = np.log(rng.uniform(0.2, 1.0, (B, H))).astype(np.float32)
    say("evict_one fill", dtype, D, Hq, "ring", ring, "append", append, "P", P)
    ev1 = torch.full((B, H, 2), -7, dtype=torch.int32, device="cuda")
    o1, l1, n1 = kvb.kv_attn_decode_evict_one(c1, to_dev(q), to_dev(t), M, k_new=to_dev(kn),
                                              v_new=to_dev(vn), log_beta_new=to_dev(lbn),
                                              num_splits=P, evicted_pos=ev1)
    o2, l2 = kvb.kv_attn_decode(c2, to_dev(q), to_dev(t), k_new=to_dev(kn), v_new=to_dev(vn),
                                log_beta_new=to_dev(lbn), num_splits=P)
    ev2 = torch.full((B, H, 2), -7, dtype=torch.int32, device="cuda")
    n2 = kvb.kv_evict_one(c2, to_dev(t), M, evicted_pos=ev2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "attention bit for bit"
    assert torch.equal(n1, n2), "n_evicted"
    n1h = to_host(n1)
    assert n1h[1, 3] == -3 and n1h[1, 1] == 0 and n1h[1, 2] == 0
    assert np.array_equal(to_host(ev1)[n1h == 1][:, 0], to_host(ev2)[n1h == 1][:, 0])
    assert np.all(to_host(ev1)[n1h != 1] == -7)
    assert torch.equal(c1.length, c2.length), "len"
    if ring:
        assert np.array_equal(to_host(c1.start), starts), "fill keeps every start"
    # the ordered result of kv_evict_one, sorted the same way, equals fill's
    a, b2 = _by_position(c1), _by_position(c2)
    ln = to_host(c1.length)
    for name in ("k", "v", "pos", "log_beta"):
        for bb in range(B):
            for g in range(H):
                m = int(ln[bb, g])
                assert np.array_equal(a[name][bb, g, :m], b2[name][bb, g, :m]), (name, bb, g)


@pytest.mark.parametrize("ring", [True, False])
def test_evict_one_fill_steady_loop(ring):
    """Decode steps at budget M with kv_attn_decode_evict_one: the slots drift out of
    position order, so ties among equal keys (one head with every log beta 0, one
    where the decode tokens carry beta = 1) must be broken by position, not slot.
    Each step's output within 2e-3 of the oracle's and the live rows, sorted by
    position, equal to the oracle's layout after every step."""
    B, H, Hq, D, M = 2, 3, 12, 128, 200
    cap = M + 4
    d = _dense(47, B, H, M, cap, D)
    d["log_beta"][0, 0, :M] = 0.0
    c = kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]), to_dev(d["pos"]),
                    to_dev(d["len"]),
                    start=torch.zeros((B, H), dtype=torch.int32, device="cuda") if ring else None)
    ref = oracle.Cache.from_arrays(d)
    rng = np.random.default_rng(9)
    for s in range(40):
        t = np.full(B, M + 3 * s, np.int32)
        kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        lbn = np.log(rng.uniform(0.3, 1.0, (B, H))).astype(np.float32)
        lbn[0, 0] = 0.0
        lbn[1, 2] = 0.0
        q = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
        o, l, ne = kvb.kv_attn_decode_evict_one(c, to_dev(q), to_dev(t), M, k_new=to_dev(kn),
                                                v_new=to_dev(vn), log_beta_new=to_dev(lbn))
        torch.cuda.synchronize()
        assert bool((ne == 1).all()), s
        oracle.append_tokens(ref, kn, vn, lbn, t)
        ro, rl = oracle_attention({"k": ref.k, "v": ref.v, "log_beta": ref.log_beta,
                                   "pos": ref.pos, "len": ref.length}, q, t)
        check_attention(to_host(o), to_host(l), ro, rl, f"fill step {s}")
        ref, _, _ = oracle.evict_to_budget(ref, t, M)
        check_layout(_by_position(c), ref, f"fill step {s}")
    pos = to_host(c.pos)
    assert not all(np.all(np.diff(pos[b, g, :M]) > 0) for b in range(B) for g in range(H)), \
        "slots should be out of position order after fill steps"


def test_evict_one_fill_full_shape_steps():
    """kv_attn_decode_evict_one at the 32K workload's model shape (batch 16, 32 query /
    8 KV heads, D = 128, M = 4096): three steps against kv_attn_decode + kv_evict_one
    on a copy: the first step's attention bit for bit (same layout), the later ones
    within 1e-4 (same tokens, other slots), every head's live rows equal as a set."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    M = w.budget
    dc = synth.device_cache(w, 0, n=M, cap=M + 32)
    B, H = w.batch, w.hkv
    c1 = kvb.KVCache.from_dict(dc)
    c2 = _copy_cache(c1)
    q, kn, vn, lbn = synth.device_queries(w, 0)
    for s in range(3):
        t = torch.full((B,), M + s, dtype=torch.int32, device="cuda")
        say("fill full shape step", s)
        o1, l1, n1 = kvb.kv_attn_decode_evict_one(c1, q, t, M, k_new=kn, v_new=vn,
                                                  log_beta_new=lbn, num_splits=16)
        o2, l2 = kvb.kv_attn_decode(c2, q, t, k_new=kn, v_new=vn, log_beta_new=lbn,
                                    num_splits=16)
        n2 = kvb.kv_evict_one(c2, t, M)
        torch.cuda.synchronize()
        if s == 0:
            assert torch.equal(o1, o2) and torch.equal(l1, l2), s
        else:
            # the same tokens in other slots: the sums run in another order
            den = o2.abs().amax(dim=-1)
            assert bool(((o1 - o2).abs().amax(dim=-1) <= 1e-4 * den).all()), s
            assert bool(((l1 - l2).abs() <= 1e-4).all()), s
        assert bool((n1 == 1).all()) and torch.equal(n1, n2), s
        a, b2 = _by_position(c1), _by_position(c2)
        for name in ("k", "v", "pos", "log_beta"):
            assert np.array_equal(a[name][:, :, :M], b2[name][:, :, :M]), (s, name)
