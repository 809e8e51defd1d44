"""In-place compaction where every kept row moves (GPU, bit-exact against the oracle).

The compaction moves rows in groups of destination rows, one group per workgroup,
with no order between groups; a source that lies inside another group's destination
range must be read before that group writes over it.  These cases make every kept
row move by a shift of 1, 2, 63, 64, 65, 127, 128, 129, ... slots (so that chains of
overlapping sources and destinations cross every group boundary, at every offset
against the group size), or by a shift that grows by one every p rows, on the erase
path, the eviction planners (one eviction, the LDS planner, the chunked selection)
and ring heads that wrap.  The oracle's layout is the out-of-place definition
(a stable filter of the rows), compared bit for bit.
"""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import check_layout, dev_cache, host_dict, say, to_dev, to_host
from test_gpu_start import _expected_start, _logical, _placed

pytestmark = pytest.mark.gpu


def _cache(seed, lens, cap, retention=True):
    lens = np.asarray(lens, np.int32)
    B, H = lens.shape
    w = synth.Workload("t", batch=B, hq=H, hkv=H, head_dim=128, dtype="bf16", ctx=int(lens.max()),
                       budget=0, layers=1, seed=seed, retention=retention)
    d = synth.host_cache(w, n=int(lens.max()), cap=cap)
    d["len"] = lens.copy()
    d["pos"] = np.broadcast_to(np.arange(cap, dtype=np.int32), (B, H, cap)).copy()
    return d


def _erase(d, per_b, what):
    B = d["len"].shape[0]
    R = max(1, max(len(x) for x in per_b))
    ranges = np.zeros((B, R, 2), np.int32)
    nr = np.zeros(B, np.int32)
    for b in range(B):
        for i, (s, e) in enumerate(per_b[b]):
            ranges[b, i] = (s, e)
        nr[b] = len(per_b[b])
    c = dev_cache(d)
    n_er = kvb.kv_erase_ranges(c, to_dev(ranges), to_dev(nr))
    torch.cuda.synchronize()
    ref, ref_n = oracle.erase_ranges(oracle.Cache.from_arrays(d),
                                     [ranges[b, :nr[b]] for b in range(B)])
    check_layout(host_dict(c), ref, what)
    assert np.array_equal(to_host(n_er), ref_n), what


@pytest.mark.parametrize("k", [1, 2, 63, 64, 65, 127, 128, 129, 1000, 4095])
def test_erase_every_row_shifts(k):
    """The first k positions erased: every kept row moves down by k slots."""
    lens = [[20000, 12345, 130, 64], [4097, 1, 9999, 20000]]
    d = _cache(700 + k, lens, 20001)
    say("erase shift", k)
    _erase(d, [[(0, k)], [(-5, k)]], f"erase shift {k}")


@pytest.mark.parametrize("p", [7, 63, 64, 65, 127, 129, 3])
def test_erase_growing_shift(p):
    """One position in every p erased: the shift grows by one every p rows, so each
    group reads from the next groups' destinations.  p = 127, 129: few enough ranges
    for the endpoint search; the others take the per-chunk scan (more ranges than
    the endpoint table holds)."""
    n = 15000 if p == 3 else 20000
    d = _cache(800 + p, [[n, n - 77], [n // 2, 333]], n + 1)
    per = [[(p * i + p - 1, p * i + p) for i in range(n // p)],
           [(p * i, p * i + 1) for i in range(1, n // p, 2)]]
    say("erase growing shift", p, [len(x) for x in per])
    _erase(d, per, f"erase every {p}")


def _evict_oldest(d, k_per_head, what):
    """log beta -1 on the k oldest slots of each head, 0 elsewhere (keys 0 there):
    eviction to n - k removes exactly them and every kept row moves down by k."""
    B, H = d["len"].shape
    t = np.full(B, int(d["len"].max()), np.int32)
    lb = np.zeros_like(d["log_beta"])
    for b in range(B):
        for g in range(H):
            lb[b, g, :k_per_head[b][g]] = -1.0
    d["log_beta"] = lb
    M = int(min(int(d["len"][b, g]) - k_per_head[b][g] for b in range(B) for g in range(H)))
    c = dev_cache(d)
    n_ev = kvb.kv_evict_to_budget(c, to_dev(t), M)
    torch.cuda.synchronize()
    ref, _, ref_n = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    check_layout(host_dict(c), ref, what)
    assert np.array_equal(to_host(n_ev), ref_n), what


@pytest.mark.parametrize("k", [1, 63, 64, 65, 129, 1000, 15000])
def test_evict_oldest_every_row_shifts(k):
    """Heads of 20000 slots (the LDS planner; the one-eviction path for k = 1) with
    the k oldest evicted."""
    lens = [[20000, 20000], [20000, 20000]]
    d = _cache(900 + k, lens, 20001)
    say("evict oldest", k)
    _evict_oldest(d, [[k, k], [k, k]], f"evict oldest {k}")


@pytest.mark.parametrize("k", [65, 4096])
def test_evict_oldest_large_heads(k):
    """Heads over the LDS planner's size (the chunked selection) with every kept row
    moving by k."""
    lens = [[40000, 40000]]
    d = _cache(950 + k, lens, 40001)
    say("evict oldest large", k)
    _evict_oldest(d, [[k, k]], f"evict oldest large {k}")


@pytest.mark.parametrize("k", [64, 65, 3000])
def test_ring_evict_middle_block(k):
    """Ring heads (a start array) that wrap around their slots, a block of k tokens
    in the middle evicted: the shorter side moves by k, across the wrap."""
    B, H, cap = 1, 4, 12000
    n = 10000
    d = _cache(990 + k, [[n] * H], n + 1)
    starts = np.array([[cap - 10, cap - 5000, 3, cap - 1]], np.int32)
    t = np.full(B, n, np.int32)
    lb = np.zeros_like(d["log_beta"])
    for g in range(H):
        ng = int(d["len"][0, g])
        mid = ng // 2 - k // 2 - (g % 2) * 7  # odd heads: the side before is shorter
        lb[0, g, mid:mid + k] = -1.0
    d["log_beta"] = lb
    M = int(d["len"].min()) - k
    c = _placed(d, starts, cap, 5 + k)
    kvb.kv_evict_to_budget(c, to_dev(t), M)
    torch.cuda.synchronize()
    ref, ref_ev, _ = oracle.evict_to_budget(oracle.Cache.from_arrays(d), t, M)
    got = _logical(c)
    assert np.array_equal(got["len"], ref.length)
    for b in range(B):
        for g in range(H):
            nk = int(ref.length[b, g])
            for name in ("k", "v", "pos", "log_beta"):
                assert np.array_equal(got[name][b, g, :nk], getattr(ref, name)[b, g, :nk]), \
                    f"ring k={k} ({b},{g}) {name}"
    assert np.array_equal(to_host(c.start), _expected_start(d, ref_ev, starts, cap)), \
        f"ring k={k} start"
