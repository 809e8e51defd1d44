"""Attention-state memory construction on the GPU against the float64 oracle.

Prefix states: every query's (a, lse) within the attention bar (2e-3 of the row's
inf-norm, lse within 2e-3).  K-means: each Lloyd iteration is checked on its own,
starting from the GPU's centroids: a point's centroid is the oracle's, or one whose
distance is within a float32 bound of the oracle's minimum (a near tie); the
update must equal the oracle mean of the GPU's assignment within float32 rounding,
with members counted exactly and empty clusters left bit for bit.  Aggregation:
the oracle merge of the GPU's clusters (abar to bf16 rounding, log Zbar 1e-5).
"""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import oracle
import synth
from gpu_util import check_attention, say, to_dev, to_host, values

pytestmark = pytest.mark.gpu


def _rne(x):
    """float32 -> bf16 bits, round to nearest even (host check of the stored copy)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _near_tie_ok(X, C, got, what, frac_exact=0.98):
    """got[n] is the nearest centroid or within a float32 bound of it."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C, np.float64)
    d2 = (C * C).sum(1)[None, :] - 2.0 * X @ C.T        # |x|^2 dropped: same for all k
    ref = np.argmin(d2, axis=1)
    exact = int((ref == got).sum())
    scale = (X * X).sum(1) + (C * C).sum(1).max()
    for n in np.nonzero(ref != got)[0]:
        g = int(got[n])
        assert 0 <= g < C.shape[0], f"{what}: point {n} label {g} out of range"
        gap = d2[n, g] - d2[n, ref[n]]
        assert gap <= 1e-5 * scale[n], f"{what}: point {n} -> {g}, oracle {ref[n]}, gap {gap:.3e}"
    assert exact >= frac_exact * X.shape[0], f"{what}: {exact} of {X.shape[0]} exact"
    return X.shape[0] - exact


def _check_update(X, C_in, assign, C_out, counts, what):
    ref = oracle.centroid_update(X, assign, C_in)
    cnt = np.bincount(assign, minlength=C_in.shape[0])
    assert np.array_equal(counts, cnt), f"{what}: member counts"
    empty = cnt == 0
    assert np.array_equal(C_out[empty].view(np.uint32),
                          np.asarray(C_in, np.float32)[empty].view(np.uint32)), \
        f"{what}: an empty cluster's centroid moved"
    den = np.abs(ref).max(1, keepdims=True) + 1e-30
    err = np.abs(C_out - ref) / den
    assert err.max() <= 1e-5, f"{what}: centroid err {err.max():.3e}"


def _check_states(a, lse, ra, rl, what):
    check_attention(a[None], lse[None], ra[None], rl[None], what)


def _inputs(H, N, L, D, seed, topics=64):
    w = synth.Workload("b", batch=1, hq=H, hkv=H, head_dim=D, dtype="bf16", ctx=max(L, 1),
                       budget=0, layers=1, seed=seed, retention=False, codebook=0)
    q, k, v = synth.host_asm_build(w, N, L, topics=topics)
    return q, k, v


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,N,L,chunks", [(1, 1, 1, 1), (2, 37, 300, 1), (2, 37, 300, 4),
                                          (1, 130, 64, 1), (2, 200, 1000, 3), (1, 129, 4097, 4),
                                          (1, 16, 70, 70)])
def test_prefix_states(D, H, N, L, chunks):
    say("prefix states", D, H, N, L, chunks)
    q, k, v = _inputs(H, N, L, D, 900 + N + L + D)
    a, lse = kvb.asm_prefix_states(to_dev(q), to_dev(k), to_dev(v), chunks=chunks)
    torch.cuda.synchronize()
    a, lse = to_host(a), to_host(lse)
    scale = 1.0 / np.sqrt(D)
    for h in range(H):
        ra, rl = oracle.prefix_states(values(q[h]), values(k[h]), values(v[h]), scale, chunks)
        _check_states(a[h], lse[h], ra, rl, f"prefix D{D} h{h} N{N} L{L} c{chunks}")


def test_prefix_states_empty_prefix_and_chunking_is_lossless():
    """L = 0 gives the empty state; 1 and 4 chunks agree to rounding (the
    online-softmax identity)."""
    q, k, v = _inputs(2, 50, 0, 128, 31)
    a, lse = kvb.asm_prefix_states(to_dev(q), to_dev(k), to_dev(v), chunks=4)
    torch.cuda.synchronize()
    assert np.all(to_host(a) == 0) and np.all(to_host(lse) == -np.inf)
    q, k, v = _inputs(2, 300, 2000, 128, 32)
    a1, l1 = kvb.asm_prefix_states(to_dev(q), to_dev(k), to_dev(v), chunks=1)
    a4, l4 = kvb.asm_prefix_states(to_dev(q), to_dev(k), to_dev(v), chunks=4)
    torch.cuda.synchronize()
    a1, l1, a4, l4 = map(to_host, (a1, l1, a4, l4))
    # the weights enter the value product rounded to fp16 relative to each chunking's
    # running maximum, so the two agree to that rounding (each is within the 2e-3 bar
    # of the oracle); the normalisers are summed unrounded
    err = np.abs(a1 - a4).max(-1) / np.abs(a1).max(-1)
    assert err.max() <= 1e-3 and np.abs(l1 - l4).max() <= 1e-5


def test_prefix_states_value_range():
    """The value product runs in fp16 with V scaled per (chunk, dimension) by a power
    of two, so values far beyond fp16's range give the oracle's states: single large
    entries, a whole dimension near bf16's top and one far below it; each dimension
    is checked against its own scale (2e-3 of its largest |value| over the queries),
    the status word stays KVB_OK.  A non-finite v sets it to KVB_ERANGE."""
    q, k, v = _inputs(1, 40, 300, 128, 55)
    ws = torch.zeros(kvb.asm_prefix_states_workspace(1, 40, 128, 300, 2), dtype=torch.uint8,
                     device="cuda")
    kvb.asm_prefix_states(to_dev(q), to_dev(k), to_dev(v), chunks=2, ws=ws)
    torch.cuda.synchronize()
    assert int(to_host(ws[:4]).view(np.int32)[0]) == 0
    vv = values(v[0]).copy()
    vv[17, 5] = 1.0e5
    vv[200, 9] = -3.0e6
    vv[:, 7] *= 1.0e37                       # every key, near the top of bf16's range
    vv[:, 70] *= 1.0e-30                     # every key, far below fp16's normal range
    vv[:150, 100] *= 7.0e4                   # one chunk only
    v2 = synth.bf16_bits(vv)[None]
    a, lse = kvb.asm_prefix_states(to_dev(q), to_dev(k), to_dev(v2), chunks=2, ws=ws)
    torch.cuda.synchronize()
    assert int(to_host(ws[:4]).view(np.int32)[0]) == 0, "no saturation"
    ra, rl = oracle.prefix_states(values(q[0]), values(k[0]), values(v2[0]), 1 / np.sqrt(128), 2)
    a, lse = to_host(a)[0].astype(np.float64), to_host(lse)[0]
    assert np.all(np.isfinite(a))
    scale = np.abs(ra).max(axis=0)           # per dimension over the queries
    err = (np.abs(a - ra) / np.maximum(scale, 1e-300)[None, :]).max()
    assert err <= 2e-3, f"per-dimension relative error {err:.3e}"
    assert np.abs(lse - rl).max() <= 2e-3
    v3 = v.copy()
    v3[0, 10, 3] = synth.bf16_bits(np.array([np.inf]))[0]
    kvb.asm_prefix_states(to_dev(q), to_dev(k), to_dev(v3), chunks=2, ws=ws)
    torch.cuda.synchronize()
    assert int(to_host(ws[:4]).view(np.int32)[0]) == -7, "non-finite v reported"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,N,K", [(1, 1, 1), (2, 300, 7), (2, 1000, 64), (1, 2500, 300),
                                   (3, 700, 1000)])
def test_kmeans_iterations(D, H, N, K):
    """Each iteration from the GPU's own centroids: assignment (near ties allowed),
    update (float32 rounding), counts exact, bf16 copy = RNE of the float32 result,
    and a second run repeats every bit."""
    say("kmeans", D, H, N, K)
    q, _, _ = _inputs(H, N, 1, D, 700 + N + K + D, topics=max(1, K // 3))
    X = values(q)
    rng = np.random.default_rng(N + K)
    init = np.stack([X[h][rng.choice(N, size=K, replace=K > N)] for h in range(H)])
    init = init.astype(np.float32)
    dx = to_dev(q)
    cent = to_dev(init.copy())
    for it in range(4):
        C_in = to_host(cent).copy()
        cb = torch.empty((H, K, D), dtype=torch.bfloat16, device="cuda")
        assign, counts, _ = kvb.asm_kmeans(dx, cent, 1, centroids_bf16=cb)
        torch.cuda.synchronize()
        A, Cn, Co = to_host(assign), to_host(counts), to_host(cent)
        for h in range(H):
            _near_tie_ok(X[h], C_in[h], A[h], f"kmeans D{D} it{it} h{h}")
            _check_update(X[h], C_in[h], A[h], Co[h], Cn[h], f"kmeans D{D} it{it} h{h}")
        assert np.array_equal(to_host(cb), _rne(Co)), "bf16 copy is not RNE of the result"
    cent2 = to_dev(init.copy())
    cent3 = to_dev(init.copy())
    a2, _, _ = kvb.asm_kmeans(dx, cent2, 4)
    a3, _, _ = kvb.asm_kmeans(dx, cent3, 4)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(a2), to_host(a3))
    assert np.array_equal(to_host(cent2).view(np.uint32), to_host(cent3).view(np.uint32))
    assert np.array_equal(to_host(cent2).view(np.uint32), to_host(cent).view(np.uint32)), \
        "4 iterations in one call differ from 4 calls of one"


def test_kmeans_separated_matches_oracle_run():
    """Well-separated clusters: the whole run equals the oracle's (no near ties)."""
    rng = np.random.default_rng(5)
    H, K, D, per = 2, 40, 128, 25
    cen = rng.standard_normal((H, K, D)) * 4.0
    lab = rng.integers(0, K, size=(H, K * per))
    X = cen[np.arange(H)[:, None], lab] + 0.05 * rng.standard_normal((H, K * per, D))
    q = synth.bf16_bits(X)
    Xv = values(q)
    init = np.stack([Xv[h][rng.choice(K * per, size=K, replace=False)] for h in range(H)])
    cent = to_dev(init.astype(np.float32))
    assign, counts, _ = kvb.asm_kmeans(to_dev(q), cent, 6)
    torch.cuda.synchronize()
    for h in range(H):
        ra, rc = oracle.kmeans(Xv[h], init[h].astype(np.float32).astype(np.float64), 6)
        assert np.array_equal(to_host(assign)[h], ra)
        err = np.abs(to_host(cent)[h] - rc).max() / np.abs(rc).max()
        assert err <= 1e-5


def test_kmeans_one_giant_cluster_and_empty_clusters():
    """All points nearest one centroid (a long member list) and the rest empty."""
    rng = np.random.default_rng(9)
    H, N, K, D = 1, 5000, 70, 128
    X = rng.standard_normal((H, N, D)) * 0.1
    q = synth.bf16_bits(X)
    init = np.concatenate([np.zeros((H, 1, D)), 50 + rng.standard_normal((H, K - 1, D))], axis=1)
    init = init.astype(np.float32)
    cent = to_dev(init.copy())
    assign, counts, _ = kvb.asm_kmeans(to_dev(q), cent, 2)
    torch.cuda.synchronize()
    assert np.all(to_host(assign) == 0)
    assert to_host(counts)[0, 0] == N and np.all(to_host(counts)[0, 1:] == 0)
    _check_update(values(q)[0], init[0], to_host(assign)[0], to_host(cent)[0], to_host(counts)[0],
                  "giant cluster")


@pytest.mark.parametrize("D", [64, 128])
def test_aggregate_states(D):
    """Random states and labels: empty clusters, labels out of range, members with
    lse = -inf, a cluster of only such members, long and short clusters."""
    rng = np.random.default_rng(D)
    H, N, K = 2, 3000, 150
    a = rng.standard_normal((H, N, D)).astype(np.float32)
    lse = rng.uniform(-20, 40, (H, N)).astype(np.float32)
    assign = rng.integers(0, K - 10, size=(H, N)).astype(np.int32)   # clusters K-10.. empty
    assign[:, :400] = 3                                              # a long cluster
    assign[0, 500] = K + 5                                           # no cluster
    assign[1, 501] = -2
    lse[0, 600:620] = -np.inf
    assign[0, 600:620] = K - 10                                      # only -inf members
    lse[1, 700] = -np.inf
    a[:, 600:620] = 0
    a[1, 700] = 0
    abar, lz = kvb.asm_aggregate_states(to_dev(assign), to_dev(a), to_dev(lse), K)
    torch.cuda.synchronize()
    abar, lz = to_host(abar), to_host(lz)
    for h in range(H):
        m = (assign[h] >= 0) & (assign[h] < K)
        lab = np.where(m, assign[h], K)                               # K: outside every cluster
        ra, rl = oracle.aggregate_states(lab, a[h].astype(np.float64), lse[h].astype(np.float64),
                                         K)
        _check_agg_arrays(abar[h], lz[h], ra, rl, f"aggregate D{D} h{h}")
    abar2, lz2 = kvb.asm_aggregate_states(to_dev(assign), to_dev(a), to_dev(lse), K)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(abar2), abar) and np.array_equal(to_host(lz2).view(np.uint32),
                                                                   lz.view(np.uint32))


def _check_agg_arrays(abar, lz, ra, rl, what):
    got = values(abar)
    for k in range(ra.shape[0]):
        if rl[k] == -np.inf:
            assert lz[k] == -np.inf and np.all(abar[k] == 0), f"{what}: empty cluster {k}"
            continue
        den = np.abs(ra[k]).max()
        err = np.abs(got[k] - ra[k]).max() / max(den, 1e-30)
        assert err <= 2 ** -8 + 1e-5, f"{what}: cluster {k} abar err {err:.3e}"
        assert abs(lz[k] - rl[k]) <= 1e-5 * max(1.0, abs(rl[k])), f"{what}: cluster {k} log Z"


def test_build_memory_small():
    """The whole build: states in the workspace, final centroids = member means of
    the last assignment, codebook = oracle aggregation of that assignment; the
    memory then answers lookups."""
    H, N, L, D, K, chunks, iters = 2, 900, 700, 128, 48, 3, 5
    q, k, v = _inputs(H, N, L, D, 77, topics=16)
    X = values(q)
    rng = np.random.default_rng(3)
    init = np.stack([X[h][rng.choice(N, size=K, replace=False)] for h in range(H)])
    cent = to_dev(init.astype(np.float32))
    cb, abar, lz, assign, ws = kvb.asm_build_memory(to_dev(q), to_dev(k), to_dev(v), cent, iters,
                                                    chunks=chunks)
    torch.cuda.synchronize()
    wsb = to_host(ws)
    off_l = 256 + ((H * N * D * 4 + 255) // 256) * 256
    a = wsb[256:256 + H * N * D * 4].view(np.float32).reshape(H, N, D)
    lse = wsb[off_l:off_l + H * N * 4].view(np.float32).reshape(H, N)
    A, C = to_host(assign), to_host(cent)
    assert np.array_equal(to_host(cb), _rne(C))
    for h in range(H):
        ra, rl = oracle.prefix_states(X[h], values(k[h]), values(v[h]), 1 / np.sqrt(D), chunks)
        _check_states(a[h], lse[h], ra, rl, f"build states h{h}")
        cnt = np.bincount(A[h], minlength=K)
        for c in np.nonzero(cnt)[0]:
            ref = X[h][A[h] == c].mean(0)
            assert np.abs(C[h, c] - ref).max() <= 1e-5 * np.abs(ref).max()
        _check_agg_arrays(to_host(abar)[h], to_host(lz)[h],
                          *oracle.aggregate_states(A[h], ra, rl, K), f"build aggregate h{h}")
        ro, rc = oracle.kmeans(X[h], init[h].astype(np.float32).astype(np.float64), iters)
        agree = (ro == A[h]).mean()
        say("build h", h, "agreement with the oracle run", agree)
        assert agree >= 0.9
    # the built memory answers lookups (group of 4 query heads per KV head)
    B, Hq = 3, 4 * H
    qq = synth.bf16_bits(rng.standard_normal((B, Hq, D)))
    so = rng.standard_normal((B, Hq, D)).astype(np.float32)
    sl = rng.uniform(-5, 5, (B, Hq)).astype(np.float32)
    out, ol, idx = kvb.asm_lookup_merge(to_dev(qq), cb, abar, lz, to_dev(so), to_dev(sl))
    torch.cuda.synchronize()
    ab = values(to_host(abar))
    lzh = to_host(lz)
    ro = np.zeros((B, Hq, D))
    rl2 = np.zeros((B, Hq))
    for b in range(B):
        for hq in range(Hq):
            i = int(to_host(idx)[b, hq])
            ro[b, hq], rl2[b, hq] = oracle.asm_merge(so[b, hq], sl[b, hq], ab[hq // 4, i],
                                                     float(lzh[hq // 4, i]))
    check_attention(to_host(out), to_host(ol), ro, rl2, "lookup on the built memory")


def test_build_full_size_sampled():
    """The memory-build workload (8 KV heads, 16K calibration queries, 16K-token
    prefix in 4 chunks, 4096 entries, 10 iterations) in the launch configuration
    the benchmark times; checked on sampled queries, points and clusters at every
    iteration."""
    w = synth.WORKLOADS["asm_build"]
    H, N, L, D, K = w.hkv, synth.BUILD_N, w.ctx, w.head_dim, w.codebook
    say("build full size")
    q, k, v = synth.host_asm_build(w, N)
    init = synth.host_kmeans_init(w, q, K)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    a, lse = kvb.asm_prefix_states(dq, dk, dv, chunks=synth.BUILD_CHUNKS)
    torch.cuda.synchronize()
    a_h, l_h = to_host(a), to_host(lse)
    rng = np.random.default_rng(1)
    for h in range(H):
        ns = rng.choice(N, size=8, replace=False)
        ra, rl = oracle.prefix_states(values(q[h, ns]), values(k[h]), values(v[h]),
                                      1 / np.sqrt(D), synth.BUILD_CHUNKS)
        _check_states(a_h[h, ns], l_h[h, ns], ra, rl, f"full-size states h{h}")
    cent = to_dev(init.copy())
    X = values(q)
    ws = torch.empty(kvb.asm_kmeans_workspace(H, K, D), dtype=torch.uint8, device="cuda")
    for it in range(synth.BUILD_ITERS):
        C_in = to_host(cent).copy()
        assign, counts, _ = kvb.asm_kmeans(dq, cent, 1, ws=ws)
        torch.cuda.synchronize()
        A, Cn, Co = to_host(assign), to_host(counts), to_host(cent)
        h = it % H
        ps = rng.choice(N, size=256, replace=False)
        _near_tie_ok(X[h, ps], C_in[h], A[h, ps], f"full-size it{it}", frac_exact=0.95)
        assert np.array_equal(Cn[h], np.bincount(A[h], minlength=K))
        for c in rng.choice(K, size=16, replace=False):
            mem = A[h] == c
            if mem.any():
                ref = X[h][mem].mean(0)
                assert np.abs(Co[h, c] - ref).max() <= 1e-5 * np.abs(ref).max()
            else:
                assert np.array_equal(Co[h, c].view(np.uint32), C_in[h, c].view(np.uint32))
    abar, lz = kvb.asm_aggregate_states(assign, a, lse, K)
    torch.cuda.synchronize()
    A, ab, lzh = to_host(assign), to_host(abar), to_host(lz)
    for h in range(H):
        cs = rng.choice(K, size=8, replace=False)
        for c in cs:
            mem = np.nonzero(A[h] == c)[0]
            ra, rl = oracle.aggregate_states(np.zeros(mem.size, np.int64), a_h[h, mem].astype(
                np.float64), l_h[h, mem].astype(np.float64), 1)
            _check_agg_arrays(ab[h, c:c + 1], lzh[h, c:c + 1], ra, rl, f"full-size agg h{h} c{c}")
