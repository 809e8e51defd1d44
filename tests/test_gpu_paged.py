"""Paged cache: kv_attn_decode_paged and kv_erase_ranges_paged against the oracle
(its page-by-page erase and append, attention over the pages' token sequence)."""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import oracle.evict as OE
import synth
from gpu_util import check_attention, say, to_dev, to_host, values

pytestmark = pytest.mark.gpu


def _dev(d):
    c = kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]), to_dev(d["pos"]),
                    to_dev(d["len"]))
    pg = kvb.KVPages(to_dev(d["table"]), to_dev(d["fill"]), to_dev(d["n_pages"]))
    return c, pg


def _host(d):
    c = OE.Cache(d["k"].copy(), d["v"].copy(),
                 None if d["log_beta"] is None else d["log_beta"].copy(), d["pos"].copy(),
                 d["len"].copy())
    return c, OE.Pages(d["table"].copy(), d["fill"].copy(), d["n_pages"].copy())


def _check_pages(c, pg, ref, rpg, what):
    """Page arrays (live entries), len, and every row of the cache arrays bit for bit
    (rows the oracle leaves alone must be left alone too)."""
    n = to_host(pg.n_pages)
    assert np.array_equal(n, rpg.n_pages), f"{what} n_pages {n} vs {rpg.n_pages}"
    tab, fil = to_host(pg.table), to_host(pg.fill)
    B, H = n.shape
    for b in range(B):
        for g in range(H):
            m = int(n[b, g])
            assert np.array_equal(tab[b, g, :m], rpg.table[b, g, :m]), f"{what} table ({b},{g})"
            assert np.array_equal(fil[b, g, :m], rpg.fill[b, g, :m]), f"{what} fill ({b},{g})"
    assert np.array_equal(to_host(c.length), ref.length), f"{what} len"
    for name in ("k", "v", "pos", "log_beta"):
        a = getattr(ref, name)
        if a is None:
            continue
        got = to_host(getattr(c, name))
        if not np.array_equal(got.view(np.uint8), a.view(np.uint8)):
            bad = np.argwhere(np.any((got != a).reshape(B, H, a.shape[2], -1), axis=3))
            raise AssertionError(f"{what} {name} differs at {bad[:8].tolist()}")


def _view_dict(c, pg):
    v = OE.paged_view(c, pg)
    return {"k": v.k, "v": v.v, "log_beta": v.log_beta, "pos": v.pos, "len": v.length}


def _attend_case(seed, G, retention, n_pages_max, max_pages, phys, num_splits, token,
                 spare_mode="some", full_fill=0.5):
    rng = np.random.default_rng(seed)
    B, H, D = 2, 2, 128
    d = synth.host_paged(rng, B, H, D, n_pages_max, max_pages, phys, retention, full_fill)
    say(f"paged attend seed={seed} G={G} lb={retention} pages<={n_pages_max} "
        f"max={max_pages} phys={phys} P={num_splits} token={token} spare={spare_mode}")
    q = synth.bf16_bits(rng.standard_normal((B, G * H, D)))
    t = np.array([int(d["pos"][b].max()) + 3 for b in range(B)], np.int32)
    c, pg = _dev(d)
    hc, hpg = _host(d)
    kw = {}
    stored = np.ones((B, H), bool)
    if token:
        kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        ln = (rng.uniform(-0.5, 0.0, (B, H)).astype(np.float32) if retention else None)
        # a free physical page per head: one no page of the head uses, or none
        spare = np.full((B, H), -1, np.int32)
        for b in range(B):
            for g in range(H):
                used = set(d["table"][b, g, :d["n_pages"][b, g]].tolist())
                free = [p for p in range(phys) if p not in used]
                if free and (spare_mode == "all" or (spare_mode == "some" and (b + g) % 3 != 2)):
                    spare[b, g] = free[int(rng.integers(0, len(free)))]
        kw = dict(k_new=to_dev(kn), v_new=to_dev(vn), log_beta_new=to_dev(ln),
                  spare=to_dev(spare))
        # the oracle attends over the sequence with the token where it was stored
        stored = OE.paged_append(hc, hpg, kn, vn, ln, t, spare)
    # a head without room attends over its cached tokens alone (the oracle's append
    # leaves it as it was)
    ref = _view_dict(hc, hpg)
    out, lse = kvb.kv_attn_decode_paged(c, pg, to_dev(q), to_dev(t), num_splits=num_splits, **kw)
    if token and not stored.all():
        with pytest.raises(kvb.KVBError):
            kvb.kv_attn_decode_paged(*_dev(d), to_dev(q), to_dev(t), num_splits=num_splits,
                                     check_status=True, **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_attention(values(ref["k"]), values(ref["v"]), ref["log_beta"],
                                     ref["pos"], ref["len"], values(q), t)
    check_attention(to_host(out), to_host(lse), ro, rl, f"paged seed={seed}")
    _check_pages(c, pg, hc, hpg, f"paged append seed={seed}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("retention", [True, False])
def test_paged_attention_vs_oracle(G, retention):
    _attend_case(100 + G, G, retention, n_pages_max=9, max_pages=12, phys=14, num_splits=3,
                 token=False)
    _attend_case(200 + G, G, retention, n_pages_max=9, max_pages=12, phys=14, num_splits=0,
                 token=True)


@pytest.mark.parametrize("num_splits", [1, 2, 5, 64])
def test_paged_attention_splits(num_splits):
    """Splits with no page, one page, and (P = 1) more than 64 pages per split (the
    page list is reloaded every 64 pages)."""
    _attend_case(300 + num_splits, 4, True, n_pages_max=150, max_pages=160, phys=170,
                 num_splits=num_splits, token=True)


def test_paged_append_room_cases():
    """Decode token: into the last page (room), onto the free page (full last page),
    or refused (no free page): KVB_ECAPACITY and the token not attended."""
    _attend_case(401, 2, True, n_pages_max=4, max_pages=6, phys=8, num_splits=2, token=True,
                 spare_mode="some", full_fill=1.0)
    _attend_case(402, 2, True, n_pages_max=4, max_pages=6, phys=8, num_splits=2, token=True,
                 spare_mode="all", full_fill=1.0)
    _attend_case(403, 8, False, n_pages_max=4, max_pages=6, phys=8, num_splits=0, token=True,
                 spare_mode="all", full_fill=0.0)
    # a full table: no room even with a free page
    _attend_case(404, 1, True, n_pages_max=4, max_pages=4, phys=8, num_splits=1, token=True,
                 spare_mode="all", full_fill=1.0)


def _erase_case(seed, n_pages_max, max_pages, phys, n_ranges, retention=True, D=128,
                aligned=False):
    rng = np.random.default_rng(seed)
    B, H = 2, 3
    d = synth.host_paged(rng, B, H, D, n_pages_max, max_pages, phys, retention)
    say(f"paged erase seed={seed} pages<={n_pages_max} max={max_pages} ranges={n_ranges} "
        f"aligned={aligned}")
    top = int(d["pos"].max()) + 5
    R = max(n_ranges, 1)
    ranges = np.zeros((B, R, 2), np.int32)
    nr = np.zeros(B, np.int32)
    hr = []
    for b in range(B):
        if aligned:
            # ranges that start and end on page boundaries of head (b, 0)
            starts = [int(d["pos"][b, 0, 32 * d["table"][b, 0, i]])
                      for i in range(d["n_pages"][b, 0])] + [top]
            cut = np.sort(rng.choice(len(starts), size=min(2 * n_ranges, len(starts) // 2 * 2),
                                     replace=False))
            edges = np.array([starts[i] for i in cut], np.int64)
        else:
            edges = np.sort(rng.choice(top, size=2 * n_ranges, replace=False))
        rr = edges.reshape(-1, 2).astype(np.int32)
        ranges[b, :rr.shape[0]] = rr
        nr[b] = rr.shape[0]
        hr.append(rr.astype(np.int64))
    c, pg = _dev(d)
    hc, hpg = _host(d)
    n_er = kvb.kv_erase_ranges_paged(c, pg, to_dev(ranges), to_dev(nr))
    torch.cuda.synchronize()
    rc, rpg, rn = OE.erase_pages(hc, hpg, hr)
    assert np.array_equal(to_host(n_er), rn), f"n_erased {to_host(n_er)} vs {rn}"
    _check_pages(c, pg, rc, rpg, f"paged erase seed={seed}")
    return d, rc, rpg


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_paged_erase_vs_oracle(seed):
    _erase_case(500 + seed, n_pages_max=10, max_pages=12, phys=14, n_ranges=4)


def test_paged_erase_many_pages_and_ranges():
    """More than one workgroup of pages per head (the new index of a workgroup's
    first surviving page sums the ones before it), hundreds of ranges."""
    _erase_case(601, n_pages_max=700, max_pages=720, phys=740, n_ranges=300)
    _erase_case(602, n_pages_max=600, max_pages=1030, phys=620, n_ranges=3, retention=False)
    # more ranges than the classification keeps in LDS: searched in global memory
    _erase_case(603, n_pages_max=300, max_pages=300, phys=310, n_ranges=1100)


def test_paged_erase_aligned_moves_nothing():
    """Ranges on page boundaries drop whole pages: no page survives in part."""
    d, rc, rpg = _erase_case(701, n_pages_max=40, max_pages=40, phys=44, n_ranges=6,
                             aligned=True)
    for b in range(2):
        old = {int(d["table"][b, 0, i]): int(d["fill"][b, 0, i])
               for i in range(d["n_pages"][b, 0])}
        for i in range(rpg.n_pages[b, 0]):
            assert rpg.fill[b, 0, i] == old[int(rpg.table[b, 0, i])], "a page survived in part"


def test_paged_erase_edge_cases():
    """No ranges (identity), a range over everything (every page leaves), float32
    rows of D = 64, empty heads."""
    _erase_case(801, n_pages_max=6, max_pages=8, phys=9, n_ranges=0)
    rng = np.random.default_rng(802)
    d = synth.host_paged(rng, 1, 2, 128, 6, 8, 9)
    c, pg = _dev(d)
    rg = torch.tensor([[[0, 1 << 30]]], dtype=torch.int32, device="cuda")
    n_er = kvb.kv_erase_ranges_paged(c, pg, rg, torch.ones(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert to_host(pg.n_pages).tolist() == [[0, 0]] and to_host(c.length).tolist() == [[0, 0]]
    assert to_host(n_er).tolist() == d["len"].tolist()
    # float32 rows, D = 64
    rng = np.random.default_rng(803)
    d = synth.host_paged(rng, 2, 2, 64, 8, 8, 10)
    d["k"] = synth.bf16_to_f64(d["k"]).astype(np.float32)
    d["v"] = synth.bf16_to_f64(d["v"]).astype(np.float32)
    c, pg = _dev(d)
    hc, hpg = _host(d)
    rr = [np.array([[5, 40], [90, 200]], np.int64), np.array([[0, 33]], np.int64)]
    ranges = np.zeros((2, 2, 2), np.int32)
    ranges[0] = rr[0]
    ranges[1, :1] = rr[1]
    kvb.kv_erase_ranges_paged(c, pg, to_dev(ranges), to_dev(np.array([2, 1], np.int32)))
    torch.cuda.synchronize()
    rc, rpg, _ = OE.erase_pages(hc, hpg, rr)
    _check_pages(c, pg, rc, rpg, "paged erase f32")


def test_paged_erase_then_decode_steps():
    """Erase, then decode steps whose tokens fill the last page and move on to free
    pages, each step's attention against the oracle's sequence."""
    d, rc, rpg = _erase_case(901, n_pages_max=8, max_pages=16, phys=20, n_ranges=3)
    rng = np.random.default_rng(902)
    B, H, D, G = 2, 3, 128, 2
    d2 = {"k": rc.k, "v": rc.v, "log_beta": rc.log_beta, "pos": rc.pos, "len": rc.length,
          "table": rpg.table, "fill": rpg.fill, "n_pages": rpg.n_pages}
    c, pg = _dev(d2)
    hc, hpg = _host(d2)
    t = np.array([int(d["pos"][b].max()) + 1 for b in range(B)], np.int32)
    for step in range(40):
        q = synth.bf16_bits(rng.standard_normal((B, G * H, D)))
        kn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        vn = synth.bf16_bits(rng.standard_normal((B, H, D)))
        ln = rng.uniform(-0.5, 0.0, (B, H)).astype(np.float32)
        spare = np.full((B, H), -1, np.int32)
        for b in range(B):
            for g in range(H):
                used = set(hpg.table[b, g, :hpg.n_pages[b, g]].tolist())
                spare[b, g] = min(p for p in range(20) if p not in used)
        stored = OE.paged_append(hc, hpg, kn, vn, ln, t, spare)
        assert stored.all()
        out, lse = kvb.kv_attn_decode_paged(c, pg, to_dev(q), to_dev(t), k_new=to_dev(kn),
                                            v_new=to_dev(vn), log_beta_new=to_dev(ln),
                                            spare=to_dev(spare), num_splits=2)
        torch.cuda.synchronize()
        ref = _view_dict(hc, hpg)
        ro, rl = oracle.decode_attention(values(ref["k"]), values(ref["v"]), ref["log_beta"],
                                         ref["pos"], ref["len"], values(q), t)
        check_attention(to_host(out), to_host(lse), ro, rl, f"paged step {step}")
        t = t + 1
    _check_pages(c, pg, hc, hpg, "paged steps")


def test_paged_memento_full_size():
    """The 1M-slot MEMENTO trace laid out with every block and memento on fresh
    pages: erase the completed blocks (whole pages, no row moves), append the
    decode token, attend; sampled heads against the oracle."""
    w = synth.WORKLOADS["memento_1m"]
    blocks, ranges = synth.memento_layout(total=w.ctx, seed=w.seed)
    table, fill, pos0, phys = synth.memento_pages(blocks, w.hkv, seed=w.seed)
    n = table.shape[1]
    say("paged memento pages", n, "phys", phys, "ranges", ranges.shape)
    cap = 32 * phys
    dc = synth.device_cache(w, layer=0, n=cap, cap=cap)
    pos = np.zeros((w.hkv, cap), np.int32)
    for g in range(w.hkv):
        for i in range(n):
            pos[g, 32 * table[g, i]:32 * table[g, i] + fill[i]] = pos0[i] + np.arange(fill[i])
    dc["pos"].copy_(torch.from_numpy(pos[None]))
    dc["len"].fill_(int(fill.sum()))
    c = kvb.KVCache.from_dict(dc)
    mp = n + 8
    tab = np.full((1, w.hkv, mp), -1, np.int32)
    tab[0, :, :n] = table
    fil = np.zeros((1, w.hkv, mp), np.int32)
    fil[0, :, :n] = fill
    pg = kvb.KVPages(to_dev(tab), to_dev(fil), to_dev(np.full((1, w.hkv), n, np.int32)))
    # pages that stay: those whose first position lies in no range
    erased = np.zeros(n, bool)
    for s, e in ranges:
        erased |= (pos0 >= s) & (pos0 < e)
    keep = np.nonzero(~erased)[0]
    kept = int(fill[keep].sum())
    k_before = {g: to_host(c.k[0, g]) for g in (0, 5)}
    rg = torch.from_numpy(ranges[None].copy()).cuda()
    nr = torch.tensor([ranges.shape[0]], dtype=torch.int32, device="cuda")
    n_er = kvb.kv_erase_ranges_paged(c, pg, rg, nr)
    torch.cuda.synchronize()
    assert (to_host(n_er) == w.ctx - kept).all()
    assert (to_host(pg.n_pages) == keep.size).all() and (to_host(c.length) == kept).all()
    th = to_host(pg.table)
    for g in range(w.hkv):
        assert np.array_equal(th[0, g, :keep.size], table[g, keep]), f"table g={g}"
        assert np.array_equal(to_host(pg.fill)[0, g, :keep.size], fill[keep])
    for g in (0, 5):
        assert np.array_equal(to_host(c.k[0, g]), k_before[g]), "a whole-page erase moved rows"
    q, kn, vn, _ = synth.device_queries(w, 0)
    t = torch.full((1,), w.ctx, dtype=torch.int32, device="cuda")
    free = [min(set(range(phys)) - set(table[g].tolist())) for g in range(w.hkv)]
    spare = torch.tensor([free], dtype=torch.int32, device="cuda")
    out, lse = kvb.kv_attn_decode_paged(c, pg, q, t, k_new=kn, v_new=vn, spare=spare,
                                        check_status=True)
    torch.cuda.synchronize()
    assert (to_host(c.length) == kept + 1).all()
    G = w.group
    oh, lh, qh = to_host(out), to_host(lse), to_host(q)
    knh, vnh = to_host(kn), to_host(vn)
    for g in (0, 5):
        rows = np.concatenate([np.arange(32 * table[g, i], 32 * table[g, i] + fill[i])
                               for i in keep])
        kk = np.concatenate([k_before[g][rows], knh[0, g][None]])[None, None]
        vv = np.concatenate([to_host(c.v[0, g])[rows], vnh[0, g][None]])[None, None]
        pp = np.concatenate([pos[g][rows], [w.ctx]])[None, None]
        ro, rl = oracle.decode_attention(values(kk), values(vv), None, pp,
                                         np.array([[kept + 1]]),
                                         values(qh[:, g * G:(g + 1) * G]), np.array([w.ctx]))
        check_attention(oh[:, g * G:(g + 1) * G], lh[:, g * G:(g + 1) * G], ro, rl,
                        f"paged memento attention g={g}")
    del dc, c
    torch.cuda.empty_cache()


def test_paged_erase_and_attention_graph_replay():
    """The erase and the attention with its decode token captured in one HIP graph
    on a user stream: every replay (inputs restored eagerly in between, queries
    redrawn) equals the eager calls bit for bit, page arrays and rows included."""
    rng = np.random.default_rng(1101)
    B, H, D, G = 2, 2, 128, 4
    d = synth.host_paged(rng, B, H, D, 9, 14, 16)
    top = int(d["pos"].max()) + 5
    ranges = np.zeros((B, 3, 2), np.int32)
    for b in range(B):
        ranges[b] = np.sort(rng.choice(top, size=6, replace=False)).reshape(3, 2)
    nr = to_dev(np.array([3, 3], np.int32))
    rg = to_dev(ranges)
    t = to_dev(np.array([top + 1, top + 2], np.int32))
    kn = to_dev(synth.bf16_bits(rng.standard_normal((B, H, D))))
    vn = to_dev(synth.bf16_bits(rng.standard_normal((B, H, D))))
    ln = to_dev(rng.uniform(-0.5, 0.0, (B, H)).astype(np.float32))
    spare = np.full((B, H), -1, np.int32)
    for b in range(B):
        for g in range(H):
            used = set(d["table"][b, g, :d["n_pages"][b, g]].tolist())
            spare[b, g] = min(p for p in range(16) if p not in used)
    spare = to_dev(spare)
    c, pg = _dev(d)
    pristine = {n: x.clone() for n, x in (("k", c.k), ("v", c.v), ("lb", c.log_beta),
                                          ("pos", c.pos), ("len", c.length), ("tab", pg.table),
                                          ("fill", pg.fill), ("np", pg.n_pages))}
    live = {"k": c.k, "v": c.v, "lb": c.log_beta, "pos": c.pos, "len": c.length,
            "tab": pg.table, "fill": pg.fill, "np": pg.n_pages}
    q = torch.empty((B, G * H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, G * H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, G * H), dtype=torch.float32, device="cuda")
    n_er = torch.empty((B, H), dtype=torch.int32, device="cuda")
    ws_e = torch.empty(kvb.kv_erase_paged_workspace(c, pg), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(kvb.kv_attn_decode_workspace(c, G * H, 0), dtype=torch.uint8,
                       device="cuda")
    user = torch.cuda.Stream()

    def restore():
        for n, x in live.items():
            x.copy_(pristine[n])

    def calls():
        kvb.kv_erase_ranges_paged(c, pg, rg, nr, n_erased=n_er, ws=ws_e, stream=user)
        kvb.kv_attn_decode_paged(c, pg, q, t, k_new=kn, v_new=vn, log_beta_new=ln, spare=spare,
                                 out=out, lse=lse, ws=ws_a, stream=user)

    def snapshot():
        return {n: x.clone() for n, x in live.items()} | {"out": out.clone(), "lse": lse.clone(),
                                                         "n_er": n_er.clone()}

    def eager():
        restore()
        torch.cuda.synchronize()
        calls()
        user.synchronize()
        return snapshot()

    q.copy_(to_dev(synth.bf16_bits(rng.standard_normal((B, G * H, D)))))
    torch.cuda.synchronize()
    ref = eager()
    # the eager result against the oracle (erase, append, attention)
    hc, hpg = _host(d)
    rc, rpg, rn = OE.erase_pages(hc, hpg, [ranges[b].astype(np.int64) for b in range(B)])
    assert np.array_equal(to_host(ref["n_er"]), rn)
    assert OE.paged_append(rc, rpg, to_host(kn), to_host(vn), to_host(ln), to_host(t),
                           to_host(spare)).all()
    v = _view_dict(rc, rpg)
    ro, rl = oracle.decode_attention(values(v["k"]), values(v["v"]), v["log_beta"], v["pos"],
                                     v["len"], values(to_host(q)), to_host(t))
    check_attention(to_host(ref["out"]), to_host(ref["lse"]), ro, rl, "paged graph eager")
    restore()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(user):
        with torch.cuda.graph(graph, stream=user):
            calls()
    torch.cuda.synchronize()
    for r in range(3):
        say("paged graph replay", r)
        q.copy_(to_dev(synth.bf16_bits(rng.standard_normal((B, G * H, D)))))
        want = eager()
        restore()
        out.fill_(float("nan"))
        n_er.fill_(-1)
        torch.cuda.synchronize()
        with torch.cuda.stream(user):
            graph.replay()
        user.synchronize()
        got = snapshot()
        for n in want:
            assert torch.equal(got[n], want[n]), f"replay {r}: {n}"


def test_paged_attention_full_size_32k():
    """The 32K layer in 1024 full pages per head on a random permutation of the
    physical pages (the launch configuration `bench.py --paged` times): identical
    to the contiguous attention over the same tokens, and two heads' query groups
    against the oracle."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    n, npg = w.ctx, w.ctx // 32
    phys = npg + 8
    cap = 32 * phys
    dc = synth.device_cache(w, layer=0, n=cap, cap=cap)
    rng = np.random.Generator(np.random.PCG64(w.seed + 91))
    table = np.stack([rng.permutation(phys)[:npg] for _ in range(w.units)]).astype(np.int32)
    tab = torch.from_numpy(table).cuda().view(w.batch, w.hkv, npg)
    slot = (tab.long()[..., :, None] * 32 + torch.arange(32, device="cuda")).reshape(
        w.batch, w.hkv, n)
    pos = torch.zeros((w.batch, w.hkv, cap), dtype=torch.int32, device="cuda")
    pos.scatter_(2, slot, torch.arange(n, dtype=torch.int32, device="cuda").expand(
        w.batch, w.hkv, n).contiguous())
    dc["pos"].copy_(pos)
    dc["len"].fill_(n)
    c = kvb.KVCache.from_dict(dc)
    pg = kvb.KVPages(tab.contiguous(), torch.full((w.batch, w.hkv, npg), 32, dtype=torch.int32,
                                                  device="cuda"),
                     torch.full((w.batch, w.hkv), npg, dtype=torch.int32, device="cuda"))
    cont = {"k": torch.gather(dc["k"], 2, slot[..., None].expand(-1, -1, -1, w.head_dim)),
            "v": torch.gather(dc["v"], 2, slot[..., None].expand(-1, -1, -1, w.head_dim)),
            "log_beta": torch.gather(dc["log_beta"], 2, slot),
            "pos": torch.arange(n, dtype=torch.int32, device="cuda").expand(
                w.batch, w.hkv, n).contiguous(),
            "len": torch.full((w.batch, w.hkv), n, dtype=torch.int32, device="cuda")}
    cc = kvb.KVCache.from_dict({k: v.contiguous() for k, v in cont.items()})
    q, _, _, _ = synth.device_queries(w, 0)
    t = torch.full((w.batch,), n, dtype=torch.int32, device="cuda")
    op, lp = kvb.kv_attn_decode_paged(c, pg, q, t)
    oc, lc = kvb.kv_attn_decode(cc, q, t)
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc), "paged != contiguous"
    G = w.group
    qh = to_host(q)
    for b, g in ((0, 0), (11, 5)):
        ro, rl = oracle.decode_attention(values(to_host(cc.k[b, g]))[None, None],
                                         values(to_host(cc.v[b, g]))[None, None],
                                         to_host(cc.log_beta[b, g])[None, None],
                                         to_host(cc.pos[b, g])[None, None], np.array([[n]]),
                                         values(qh[b:b + 1, g * G:(g + 1) * G]), np.array([n]))
        check_attention(to_host(op)[b:b + 1, g * G:(g + 1) * G],
                        to_host(lp)[b:b + 1, g * G:(g + 1) * G], ro, rl, f"paged 32K ({b},{g})")
    del dc, c, cont, cc
    torch.cuda.empty_cache()


def test_check_pages_each_violation():
    """kv_check_pages: a clean paged cache has no flags; each planted violation (all
    values in bounds) sets its bit on exactly the affected head."""
    bits = kvb.CHECK_BITS

    def base():
        d = synth.host_paged(np.random.default_rng(1201), 2, 2, 128, 8, 9, 12, full_fill=0.3)
        # every head with at least three pages
        for b in range(2):
            for g in range(2):
                if d["n_pages"][b, g] < 3:
                    d2 = synth.host_paged(np.random.default_rng(1300 + 2 * b + g), 1, 1, 128, 8,
                                          9, 12, full_fill=0.3)
                    assert d2["n_pages"][0, 0] >= 3
                    for name in ("k", "v", "log_beta", "pos"):
                        d[name][b, g] = d2[name][0, 0]
                    for name in ("table", "fill"):
                        d[name][b, g] = d2[name][0, 0]
                    d["n_pages"][b, g] = d2["n_pages"][0, 0]
                    d["len"][b, g] = d2["len"][0, 0]
        return d

    def run(d, t=None):
        c, pg = _dev(d)
        f = kvb.kv_check_pages(c, pg, t=None if t is None else to_dev(t))
        torch.cuda.synchronize()
        return to_host(f)

    d = base()
    t = np.array([int(d["pos"][b].max()) + 1 for b in range(2)], np.int32)
    assert not run(d, t).any()
    cases = []
    d = base()
    d["n_pages"][0, 1] = 10                              # above max_pages (9)
    cases.append(("pages", d, None, (0, 1)))
    d = base()
    d["table"][1, 0, 1] = 12                             # physical page past cap / 32
    cases.append(("pages", d, None, (1, 0)))
    d = base()
    d["fill"][1, 1, 2] = 0                               # empty page in the table
    cases.append(("pages", d, None, (1, 1)))
    d = base()
    d["fill"][0, 0, 0] = 33                              # fill past the page
    cases.append(("pages", d, None, (0, 0)))
    d = base()
    d["len"][1, 1] += 1                                  # len is not the sum of the fills
    cases.append(("len", d, None, (1, 1)))
    d = base()
    d["table"][0, 1, 1] = d["table"][0, 1, 0]            # one physical page listed twice
    d["fill"][0, 1, 1] = d["fill"][0, 1, 0]
    d["len"][0, 1] = int(d["fill"][0, 1, :d["n_pages"][0, 1]].sum())
    cases.append(("pos_order", d, None, (0, 1)))
    d = base()
    for name in ("table", "fill"):                       # two pages out of order
        d[name][1, 0, [0, 1]] = d[name][1, 0, [1, 0]]
    cases.append(("pos_order", d, None, (1, 0)))
    d = base()
    i2 = int(np.nonzero(d["fill"][0, 0, :d["n_pages"][0, 0]] >= 2)[0][0])
    p0 = 32 * d["table"][0, 0, i2]
    d["pos"][0, 0, p0 + 1] = d["pos"][0, 0, p0]          # repeated position inside a page
    cases.append(("pos_order", d, None, (0, 0)))
    d = base()
    d["log_beta"][1, 1, 32 * d["table"][1, 1, 2]] = np.nan
    cases.append(("log_beta_nan", d, None, (1, 1)))
    d = base()
    d["log_beta"][0, 1, 32 * d["table"][0, 1, 0]] = 0.5
    cases.append(("log_beta_positive", d, None, (0, 1)))
    d = base()
    tt = np.array([int(d["pos"][0].max()) + 1, int(d["pos"][1, 0].max()) - 1], np.int32)
    both = d["pos"][1, 1].max() > tt[1]                  # head (1, 1) past t as well
    cases.append(("pos_after_t", d, tt, "b1" if both else (1, 0)))
    for name, d, tt, where in cases:
        say("check pages", name, where)
        f = run(d, tt)
        for b in range(2):
            for g in range(2):
                hit = (where == "b1" and b == 1) or where == (b, g)
                assert (f[b, g] & bits[name]) == (bits[name] if hit else 0), (name, b, g, f)
                if not hit:
                    assert f[b, g] == 0, (name, b, g, f)


def test_paged_memento_full_size_partial_pages():
    """The 1M-token MEMENTO trace in full pages (blocks not aligned to pages, so
    every erased range leaves partly erased pages at both ends): per-head counts in
    closed form for all heads; head 0's table, fills, positions and moved rows
    against the oracle's page-by-page erase (run on slot numbers in place of the
    rows, then the rows compared with the pre-erase rows they name)."""
    w = synth.WORKLOADS["memento_1m"]
    blocks, ranges = synth.memento_layout(total=w.ctx, seed=w.seed)
    n = w.ctx
    npg = n // 32
    phys = npg + 8
    cap = 32 * phys
    say("paged memento partial pages: pages", npg, "ranges", ranges.shape)
    dc = synth.device_cache(w, layer=0, n=cap, cap=cap)
    rng = np.random.Generator(np.random.PCG64(w.seed + 5))
    table = np.stack([rng.permutation(phys)[:npg] for _ in range(w.hkv)]).astype(np.int32)
    tab = torch.from_numpy(table).cuda().view(1, w.hkv, npg)
    slot = (tab.long()[..., :, None] * 32 + torch.arange(32, device="cuda")).reshape(1, w.hkv, n)
    pos = torch.zeros((1, w.hkv, cap), dtype=torch.int32, device="cuda")
    pos.scatter_(2, slot, torch.arange(n, dtype=torch.int32, device="cuda").expand(
        1, w.hkv, n).contiguous())
    dc["pos"].copy_(pos)
    dc["len"].fill_(n)
    c = kvb.KVCache.from_dict(dc)
    mp = npg + 4
    tab0 = np.full((1, w.hkv, mp), -1, np.int32)
    tab0[0, :, :npg] = table
    fil0 = np.zeros((1, w.hkv, mp), np.int32)
    fil0[0, :, :npg] = 32
    pg = kvb.KVPages(to_dev(tab0), to_dev(fil0), to_dev(np.full((1, w.hkv), npg, np.int32)))
    k_before = c.k[0, 0].clone()
    v_before = c.v[0, 0].clone()
    pos_before = to_host(c.pos[0, 0])
    rg = torch.from_numpy(ranges[None].copy()).cuda()
    nr = torch.tensor([ranges.shape[0]], dtype=torch.int32, device="cuda")
    n_er = kvb.kv_erase_ranges_paged(c, pg, rg, nr)
    torch.cuda.synchronize()
    # closed form for every head: kept tokens and the pages that keep any
    keep_tok = oracle.erase_plan(np.arange(n), n, ranges)
    kept = int(keep_tok.sum())
    pages_kept = int(keep_tok.reshape(npg, 32).any(axis=1).sum())
    assert kept == 200 * (len(blocks) - 1) + blocks[-1][1]
    assert (to_host(n_er) == n - kept).all() and (to_host(c.length) == kept).all()
    assert (to_host(pg.n_pages) == pages_kept).all()
    # head 0 against the oracle: rows replaced by their slot numbers
    hc = OE.Cache(np.arange(cap, dtype=np.int64).reshape(1, 1, cap, 1),
                  np.arange(cap, dtype=np.int64).reshape(1, 1, cap, 1), None,
                  pos_before.reshape(1, 1, cap), np.array([[n]], np.int32))
    hp = OE.Pages(tab0[:, :1].copy(), fil0[:, :1].copy(), np.array([[npg]], np.int32))
    rc, rp, rn = OE.erase_pages(hc, hp, [ranges.astype(np.int64)])
    assert rn[0, 0] == n - kept and rp.n_pages[0, 0] == pages_kept
    m = int(rp.n_pages[0, 0])
    assert np.array_equal(to_host(pg.table)[0, 0, :m], rp.table[0, 0, :m])
    assert np.array_equal(to_host(pg.fill)[0, 0, :m], rp.fill[0, 0, :m])
    live = np.concatenate([np.arange(32 * p, 32 * p + f)
                           for p, f in zip(rp.table[0, 0, :m], rp.fill[0, 0, :m])])
    assert np.array_equal(to_host(c.pos[0, 0])[live], rc.pos[0, 0, live])
    src = torch.from_numpy(rc.k[0, 0, live, 0].copy()).cuda()
    dst = torch.from_numpy(live.astype(np.int64)).cuda()
    assert torch.equal(c.k[0, 0].index_select(0, dst), k_before.index_select(0, src))
    assert torch.equal(c.v[0, 0].index_select(0, dst), v_before.index_select(0, src))
    del dc, c, k_before, v_before
    torch.cuda.empty_cache()
