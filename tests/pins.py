"""Pin checks that tie the float64 oracle to something other than itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with an
independent statement of what the pages fix: a library routine (torch's scaled
dot-product attention, scipy's logsumexp), a closed form written without logs
(beta_i ** (t - i)), an identity (online softmax, lossless merge), or brute
force over every subset on tiny inputs.  The functions are looked up through
the oracle's modules at call time, so tests/test_oracle_mutations.py can plant
mistakes in the oracle and show each one fails a pin.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import scipy.special
import torch

import oracle.asm as OA
import oracle.asm_build as OAB
import oracle.attn as OT
import oracle.bytes_model as OB
import oracle.evict as OE
import oracle.latent as OL

TOL = 1e-11


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _sdpa(q, K, V, scale, mask=None):
    """torch's scaled dot-product attention in float64 on the CPU (one query)."""
    qt = torch.tensor(q, dtype=torch.float64).reshape(1, 1, 1, -1)
    Kt = torch.tensor(K, dtype=torch.float64).reshape(1, 1, K.shape[0], -1)
    Vt = torch.tensor(V, dtype=torch.float64).reshape(1, 1, V.shape[0], -1)
    m = None if mask is None else torch.tensor(mask, dtype=torch.float64).reshape(1, 1, 1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m, scale=scale)
    return o.reshape(-1).numpy()


# ---------------------------------------------------------------- P1
def check_attention_library(seed=0):
    """beta == 1 reduces to textbook softmax attention: torch SDPA + scipy logsumexp."""
    r = _rng(seed)
    for n, D in ((1, 8), (7, 16), (37, 32), (130, 64)):
        q = r.standard_normal(D)
        K = r.standard_normal((n, D)) * 2.0
        V = r.standard_normal((n, D))
        scale = 1.0 / math.sqrt(D)
        pos = np.arange(n) * 3 + 5
        out, lse = OT.attention(q, K, V, None, pos, int(pos[-1]) + 1, scale)
        ref = _sdpa(q, K, V, scale)
        assert np.max(np.abs(out - ref)) < TOL * 10, "attention != SDPA"
        ref_lse = scipy.special.logsumexp(scale * (K @ q))
        assert abs(lse - ref_lse) < TOL * 10, "lse != logsumexp"
        # a non-default scale reaches the dot product
        out2, _ = OT.attention(q, K, V, None, pos, int(pos[-1]) + 1, 0.37)
        assert np.max(np.abs(out2 - _sdpa(q, K, V, 0.37))) < TOL * 10


# ---------------------------------------------------------------- P2
def check_bias_closed_form(seed=1):
    """Weights e^{scale q.k_i} * beta_i^(t - pos_i), renormalised, with no logs.

    Positions are gapped (slot != position) and include the decode token at
    distance 0 with beta = 0 (beta^0 = 1).
    """
    r = _rng(seed)
    for n in (1, 2, 5, 9):
        D = 8
        q = r.standard_normal(D)
        K = r.standard_normal((n, D))
        V = r.standard_normal((n, D))
        scale = 1.0 / math.sqrt(D)
        pos = np.sort(r.choice(40, size=n, replace=False)).astype(np.int64)
        t = int(pos[-1])                       # the newest token is the query token
        lb32 = np.log(r.uniform(0.4, 1.0, size=n)).astype(np.float32)
        lb32[-1] = -np.inf                     # beta = 0 at distance 0
        beta = np.exp(lb32.astype(np.float64))
        w = np.array([math.exp(scale * float(q @ K[i])) * (beta[i] ** int(t - pos[i]))
                      for i in range(n)])
        ref = (w @ V) / w.sum()
        out, lse = OT.attention(q, K, V, lb32, pos, t, scale)
        assert np.max(np.abs(out - ref)) < 1e-12, "biased attention != closed form"
        assert abs(lse - math.log(w.sum())) < 1e-12, "biased lse != closed form"


# ---------------------------------------------------------------- P3
def _rand_state(r, D, empty=False):
    if empty:
        return (np.zeros(D), -np.inf, 0.0)
    return (r.standard_normal(D), float(r.normal(0, 30)), float(r.uniform(0.5, 50)))


def check_split_merge(seed=2):
    """Online-softmax identity: any partition (empty blocks included), merged, equals
    full attention; merge is associative, commutative, and (0,-inf,0) is its identity."""
    r = _rng(seed)
    for n, D in ((1, 4), (33, 8), (200, 16)):
        q = r.standard_normal(D)
        K = r.standard_normal((n, D)) * 1.5
        V = r.standard_normal((n, D))
        pos = np.arange(n)
        t = n
        lb = np.log(r.uniform(0.8, 1.0, size=n)).astype(np.float32)
        full_o, full_l = OT.attention(q, K, V, lb, pos, t, 0.5)
        for _ in range(5):
            cuts = np.sort(r.integers(0, n + 1, size=r.integers(0, 6)))
            bounds = [0] + [int(c) for c in cuts] + [n]
            o, l, _ = OT.split_attention(q, K, V, lb, pos, t, 0.5, bounds)
            assert np.max(np.abs(o - full_o)) < TOL * 10, "split+merge != full"
            assert abs(l - full_l) < TOL * 10, "split+merge lse != full"
    D = 6
    for _ in range(20):
        A, Bs, C = (_rand_state(r, D, empty=(r.uniform() < 0.2)) for _ in range(3))
        ab_c = OT.state_to_out_lse(OT.merge_states([OT.merge_states([A, Bs]), C]))
        a_bc = OT.state_to_out_lse(OT.merge_states([A, OT.merge_states([Bs, C])]))
        ba = OT.state_to_out_lse(OT.merge_states([Bs, A]))
        ab = OT.state_to_out_lse(OT.merge_states([A, Bs]))
        assert np.allclose(ab_c[0], a_bc[0], atol=1e-12) and \
            (ab_c[1] == a_bc[1] or abs(ab_c[1] - a_bc[1]) < 1e-12), "merge not associative"
        assert np.allclose(ab[0], ba[0], atol=1e-12), "merge not commutative"
        ident = OT.state_to_out_lse(OT.merge_states([A, (np.zeros(D), -np.inf, 0.0)]))
        a_only = OT.state_to_out_lse(OT.merge_states([A]))
        assert np.allclose(ident[0], a_only[0]) and \
            (ident[1] == a_only[1]), "empty state is not the identity"
    # two explicit states against the page's formula (Z_A a_A + Z_B a_B)/(Z_A + Z_B)
    aA, aB = r.standard_normal(D), r.standard_normal(D)
    ZA, ZB = 3.0, 5.0
    o, l = OT.state_to_out_lse(OT.merge_states([(aA, 0.0, ZA), (aB, 0.0, ZB)]))
    assert np.allclose(o, (ZA * aA + ZB * aB) / (ZA + ZB), atol=1e-14)
    assert abs(l - math.log(ZA + ZB)) < 1e-14


# ---------------------------------------------------------------- P4
def check_asm_lossless(seed=3):
    """Merging a query's own state with the prefix state equals attention over
    [prefix; own tokens] (torch SDPA); log Zbar = -inf leaves the own state."""
    r = _rng(seed)
    D = 16
    scale = 1.0 / math.sqrt(D)
    for npre, nself in ((5, 3), (64, 17), (1, 1)):
        q = r.standard_normal(D)
        Kp, Vp = r.standard_normal((npre, D)), r.standard_normal((npre, D))
        Ks, Vs = r.standard_normal((nself, D)), r.standard_normal((nself, D))
        abar, lzbar = OT.attention(q, Kp, Vp, None, np.arange(npre), npre, scale)
        so, sl = OT.attention(q, Ks, Vs, None, np.arange(nself), nself, scale)
        mo, ml = OA.asm_merge(so, sl, abar, lzbar)
        ref = _sdpa(q, np.vstack([Kp, Ks]), np.vstack([Vp, Vs]), scale)
        ref_l = scipy.special.logsumexp(scale * (np.vstack([Kp, Ks]) @ q))
        assert np.max(np.abs(mo - ref)) < 1e-12, "ASM merge is not lossless"
        assert abs(ml - ref_l) < 1e-12, "ASM merge lse is not lossless"
        mo2, ml2 = OA.asm_merge(so, sl, abar, -np.inf)
        assert np.allclose(mo2, so, atol=1e-15) and abs(ml2 - sl) < 1e-15
        mo3, ml3 = OA.asm_merge(np.zeros(D), -np.inf, abar, lzbar)
        assert np.allclose(mo3, abar, atol=1e-15) and abs(ml3 - lzbar) < 1e-15


# ---------------------------------------------------------------- P5
def _score_order_key(beta, d, p):
    return (beta ** d, p)


def check_evict_bruteforce(seed=4, trials=40):
    """For n <= 10 exactly one M-subset has every kept token above every evicted one
    in (beta^(t-i), position) order, scores taken as the plain power; it must be the
    oracle's kept set."""
    r = _rng(seed)
    for _ in range(trials):
        n = int(r.integers(1, 11))
        M = int(r.integers(0, n + 1))
        pos = np.sort(r.choice(30, size=n, replace=False)).astype(np.int64)
        t = int(pos[-1]) + int(r.integers(0, 3))
        lb32 = np.log(r.uniform(0.3, 1.0, size=n)).astype(np.float32)
        if r.uniform() < 0.3:       # force ties in the score
            lb32[:] = lb32[0]
        beta = np.exp(lb32.astype(np.float64))
        keys = [_score_order_key(float(beta[i]), int(t - pos[i]), int(pos[i])) for i in range(n)]
        m_keep = min(n, M)
        good = []
        for kept in itertools.combinations(range(n), m_keep):
            ks = set(kept)
            ev = [keys[i] for i in range(n) if i not in ks]
            kp = [keys[i] for i in kept]
            if not ev or not kp or min(kp) > max(ev):
                good.append(ks)
        assert len(good) == 1, "brute force: separating subset not unique"
        keep, gone = OE.evict_plan(lb32, pos, n, t, M)
        assert set(np.nonzero(keep)[0].tolist()) == good[0], "eviction != brute force"
        assert list(gone) == sorted(pos[~keep].tolist()), "evicted positions"


def check_evict_sliding_window(seed=5):
    """beta == 1 (no array) or one shared beta: the newest M tokens stay."""
    r = _rng(seed)
    for n, M in ((10, 3), (50, 49), (7, 0), (5, 5), (5, 9), (300, 17)):
        pos = np.sort(r.choice(10 * n + 10, size=n, replace=False)).astype(np.int64)
        t = int(pos[-1]) + 1
        for lb in (None, np.full(n, np.float32(np.log(0.9)), np.float32),
                   np.zeros(n, np.float32)):
            keep, gone = OE.evict_plan(lb, pos, n, t, M)
            want = np.zeros(n, bool)
            want[max(0, n - M):] = True
            assert np.array_equal(keep, want), "sliding window"
            assert len(gone) == max(0, n - M)


def check_evict_invariants(seed=6):
    """len = min(n, M); the decode token (distance 0) stays when M >= 1; kept and
    evicted partition the live tokens; -0.0 and +0.0 are one key."""
    r = _rng(seed)
    for _ in range(30):
        n = int(r.integers(1, 200))
        M = int(r.integers(0, n + 5))
        pos = np.arange(n, dtype=np.int64)
        t = n - 1
        lb = np.log(1.0 / (1.0 + np.exp(-r.normal(2, 1.5, size=n)))).astype(np.float32)
        keep, gone = OE.evict_plan(lb, pos, n, t, M)
        assert keep.sum() == min(n, M)
        if M >= 1:
            assert keep[-1], "decode token evicted"
        assert sorted(np.concatenate([pos[keep], gone]).tolist()) == pos.tolist()
    k = OE.retention_keys(np.array([-0.5, 0.0, -0.0], np.float32), np.array([3, 1, 2]), 3)
    assert not np.signbit(k).any() and np.all(k == 0.0), "-0.0 not canonical"
    k2 = OE.retention_keys(np.array([-0.5, -0.25], np.float32), np.array([1, 2]), 3)
    assert k2.tolist() == [-1.0, -0.25], "key = (t - pos) * log beta"
    assert OE.retention_keys(None, np.array([0, 5]), 9).tolist() == [0.0, 0.0]


# ---------------------------------------------------------------- P6
def check_compaction(seed=7):
    """Compaction keeps each kept row bit for bit, in slot order; positions stay
    strictly increasing; rows are moved as raw storage values."""
    r = _rng(seed)
    B, H, cap, D = 2, 3, 40, 4
    c = OE.Cache(r.integers(0, 65535, size=(B, H, cap, D)).astype(np.uint16),
                 r.integers(0, 65535, size=(B, H, cap, D)).astype(np.uint16),
                 r.standard_normal((B, H, cap)).astype(np.float32),
                 np.tile(np.arange(cap, dtype=np.int32) * 2, (B, H, 1)),
                 np.full((B, H), 33, np.int32))
    for b in range(B):
        for g in range(H):
            keep = r.uniform(size=33) < 0.4
            before = c.copy()
            kept = OE.compact_unit(c, b, g, keep)
            idx = np.nonzero(keep)[0]
            assert kept == idx.size and c.length[b, g] == kept
            for j, s in enumerate(idx):
                assert np.array_equal(c.k[b, g, j], before.k[b, g, s])
                assert np.array_equal(c.v[b, g, j], before.v[b, g, s])
                assert c.log_beta[b, g, j].tobytes() == before.log_beta[b, g, s].tobytes()
                assert c.pos[b, g, j] == before.pos[b, g, s]
            assert np.all(np.diff(c.pos[b, g, :kept]) > 0)


# ---------------------------------------------------------------- P7
def check_erase_bruteforce(seed=8):
    """Set filter written as a plain loop; empty range list is the identity."""
    r = _rng(seed)
    for _ in range(30):
        n = int(r.integers(0, 60))
        pos = np.sort(r.choice(200, size=n, replace=False)).astype(np.int64)
        edges = np.sort(r.choice(210, size=2 * int(r.integers(0, 5)), replace=False))
        ranges = edges.reshape(-1, 2)
        keep = OE.erase_plan(pos, n, ranges)
        for i in range(n):
            inside = False
            for s, e in ranges:
                if s <= pos[i] and pos[i] < e:
                    inside = True
            assert keep[i] == (not inside), "erase != set filter"
        assert OE.erase_plan(pos, n, np.zeros((0, 2), np.int64)).all()


# ---------------------------------------------------------------- P8
def check_lookup_bruteforce(seed=9):
    """Cosine argmax written as a loop with math.sqrt; ties to the lowest index;
    q = lambda * c_j finds j; centroids of unequal length."""
    r = _rng(seed)
    for K, D in ((1, 4), (9, 8), (64, 16)):
        C = r.standard_normal((K, D)) * r.uniform(0.2, 3.0, size=(K, 1))
        if K > 3:
            C[K - 1] = C[1]                                    # duplicate: tie
        q = r.standard_normal(D)
        best, bk = -2.0, -1
        qn = math.sqrt(sum(x * x for x in q))
        for k in range(K):
            dot = sum(float(C[k, d]) * float(q[d]) for d in range(D))
            cn = math.sqrt(sum(float(x) * float(x) for x in C[k]))
            cs = dot / (cn * qn)
            if cs > best:
                best, bk = cs, k
        assert OA.cosine_lookup(q, C) == bk, "lookup != brute force"
        j = int(r.integers(0, K))
        if K > 3 and j == K - 1:
            j = 1
        assert OA.cosine_lookup(2.5 * C[j], C) == j, "q = lambda c_j"
    # a long centroid at a wider angle: the raw dot product prefers it, cosine does not
    C = np.array([[1.0, 0.0, 0.0], [10.0, 10.0, 0.0], [0.0, 0.0, 1.0]])
    assert OA.cosine_lookup(np.array([1.0, 0.1, 0.0]), C) == 0, "cosine, not dot product"
    # equal similarities: the lowest index wins
    C = np.array([[0.0, 1.0], [2.0, 0.0], [0.0, 3.0], [5.0, 0.0]])
    assert OA.cosine_lookup(np.array([1.0, 0.0]), C) == 1, "ties go to the lowest index"
    assert OA.cosine_lookup(np.array([0.0, 0.5]), C) == 0, "ties go to the lowest index"


# ---------------------------------------------------------------- P10
def check_hier_lookup(seed=10):
    """Two-level lookup: expanding every first-level cluster is the linear lookup
    (whatever the clustering and the order the entries are stored in); small
    hand-built cases fix the expansion, the tie rules and the returned index."""
    r = _rng(seed)
    for K, K1, D in ((7, 3, 4), (40, 6, 8), (96, 12, 16)):
        C = r.standard_normal((K, D)) * r.uniform(0.2, 3.0, size=(K, 1))
        C[K - 1] = C[2]                                        # duplicate entry: tie
        assign = r.integers(0, K1, size=K)
        assign[:K1] = np.arange(K1)                            # no empty cluster
        perm = np.lexsort((r.permutation(K), assign))          # cluster order, shuffled inside
        offs = np.searchsorted(assign[perm], np.arange(K1 + 1))
        c1 = r.standard_normal((K1, D))
        for _ in range(4):
            q = r.standard_normal(D)
            assert OA.hier_lookup(q, c1, offs, C[perm], perm, K1) == OA.cosine_lookup(q, C), \
                "full expansion != linear lookup"
        j = int(r.integers(0, K))
        if j == K - 1:
            j = 2
        assert OA.hier_lookup(1.7 * C[j], c1, offs, C[perm], perm, K1) == j, "q = lambda c_j"
    # clusters {e0, e0+e1}, {e2, e3}: stored (1, 0, 3, 2) -> kid = (1, 0, 3, 2)
    C = np.array([[1.0, 1.0, 0.0, 0.0], [1.0, 0.0, 0.0, 0.0],
                  [0.0, 0.0, 0.0, 1.0], [0.0, 0.0, 1.0, 0.0]])
    kid = np.array([1, 0, 3, 2])
    offs = np.array([0, 2, 4])
    c1 = np.array([[1.0, 0.5, 0.0, 0.0], [0.0, 0.0, 1.0, 1.0]])
    q = np.array([1.0, 0.2, 0.9, 0.0])
    # first level 0.72 / 0.47 keeps cluster 0, which holds the linear best e0
    # (original index 0, stored second; cos 0.74 against 0.62 for e0+e1)
    assert OA.cosine_lookup(q, C[np.argsort(kid)]) == 0
    assert OA.hier_lookup(q, c1, offs, C, kid, 1) == 0, "expanded cluster, original index"
    # first level 0.55 / 0.79 keeps cluster 1 while the linear best is e0 (cos 0.61);
    # inside cluster 1, e3 and e2 tie at 0.56: the lower original index (2) wins
    # although e3 is stored first
    q = np.array([0.55, 0.0, 0.5, 0.5])
    assert OA.cosine_lookup(q, C[np.argsort(kid)]) == 0
    assert OA.hier_lookup(q, c1, offs, C, kid, 1) == 2, "best inside the kept cluster only"
    assert OA.hier_lookup(q, c1, offs, C, kid, 2) == 0, "two clusters kept"
    # first-level centroids of unequal length: cosine keeps cluster 0 (0.92 against
    # 0.39), a raw dot product would keep cluster 1 (1.0 against 3.0)
    c1d = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 5.0, 5.0]])
    assert OA.hier_lookup(np.array([1.0, 0.0, 0.3, 0.3]), c1d, offs, C, kid, 1) == 0, \
        "first level by cosine"
    # equal first-level similarities: the lower j is kept
    c1t = np.array([[0.0, 0.0, 1.0, 0.0], [1.0, 0.0, 0.0, 0.0]])
    qt = np.array([1.0, 0.0, 1.0, 0.0])
    # (j = 0 holds e0 -> index 0; keeping j = 1 instead would give e2 -> index 2)
    assert OA.hier_lookup(qt, c1t, offs, C, kid, 1) == 0, "first-level tie -> lower j"
    # equal entry similarities inside the kept clusters: the lowest original index
    Ct = np.array([[0.0, 1.0], [0.0, 2.0], [1.0, 0.0]])
    assert OA.hier_lookup(np.array([0.0, 1.0]), np.array([[0.0, 1.0]]), np.array([0, 3]),
                          Ct, np.array([7, 4, 5]), 1) == 4, "entry tie -> lowest index"
    # a zero query gives index 0; a kept cluster without entries gives index 0
    assert OA.hier_lookup(np.zeros(4), c1, offs, C, kid, 2) == 0
    assert OA.hier_lookup(np.array([0.0, 1.0]), np.array([[0.0, 1.0], [1.0, 0.0]]),
                          np.array([0, 0, 3]), Ct, np.array([7, 4, 5]), 1) == 0


# ---------------------------------------------------------------- P11
def check_asm_build(seed=11):
    """Memory construction: chunked prefix states equal one-pass attention and a
    library attention routine; K-means on hand-checked 1-D data, its tie rule, an
    empty cluster, blob recovery and a non-increasing objective; the aggregation as
    its closed form."""
    r = _rng(seed)
    # (1) prefix states: any chunking = one pass = SDPA
    for L, D in ((1, 4), (37, 8), (200, 16)):
        Kp = r.standard_normal((L, D))
        Vp = r.standard_normal((L, D))
        Q = r.standard_normal((5, D)) * 2.0
        scale = 1.0 / math.sqrt(D)
        a1, l1 = OAB.prefix_states(Q, Kp, Vp, scale, 1)
        for ch in (2, 3, 4, L + 5):
            a2, l2 = OAB.prefix_states(Q, Kp, Vp, scale, ch)
            assert np.allclose(a1, a2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0,
                                                                            atol=1e-12)
        for i in range(Q.shape[0]):
            ref = _sdpa(Q[i], Kp, Vp, scale)
            assert np.allclose(a1[i], ref, rtol=0, atol=1e-12), "prefix state != SDPA"
            s_ = scale * (Kp @ Q[i])
            assert abs(l1[i] - scipy.special.logsumexp(s_)) < 1e-12, "prefix lse != logsumexp"
    assert OAB.chunk_bounds(10, 4) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    # (2) K-means, 1-D by hand: {0, 1, 10, 11, 12} from {0, 12} -> {0.5, 11}
    X = np.array([[0.0], [1.0], [10.0], [11.0], [12.0]])
    assign, C = OAB.kmeans(X, np.array([[0.0], [12.0]]), 3)
    assert list(assign) == [0, 0, 1, 1, 1] and np.allclose(C[:, 0], [0.5, 11.0])
    # equidistant -> lower index; a centroid with no members stays put
    assert OAB.nearest_centroid(np.array([1.0]), np.array([[0.0], [2.0]])) == 0
    assign, C = OAB.kmeans(X, np.array([[0.0], [12.0], [1000.0]]), 2)
    assert C[2, 0] == 1000.0 and not np.any(assign == 2)
    # separated blobs, one seed point in each: one iteration recovers the blobs;
    # the within-cluster sum of squares never increases
    centers = r.standard_normal((5, 8)) * 20.0
    lab = r.integers(0, 5, size=300)
    lab[:5] = np.arange(5)
    Xb = centers[lab] + r.standard_normal((300, 8))
    assign, _ = OAB.kmeans(Xb, Xb[:5], 1)
    assert np.array_equal(assign, lab), "blobs not recovered"
    Xr = r.standard_normal((120, 6))
    C = Xr[:7].copy()
    prev = np.inf
    for _ in range(6):
        assign, C = OAB.kmeans(Xr, C, 1)
        sse = float(np.sum((Xr - C[assign]) ** 2))
        assert sse <= prev + 1e-9, "K-means objective increased"
        prev = sse
    # (3) aggregation: Z-weighted mean of outputs, normalisers added
    a = r.standard_normal((4, 3))
    lse = np.array([2.0, -1.0, 0.5, -np.inf])
    assign = np.array([1, 1, 0, 0])
    abar, lz = OAB.aggregate_states(assign, a, lse, 3)
    w = np.exp(lse[:2])
    assert np.allclose(abar[1], (w[0] * a[0] + w[1] * a[1]) / (w[0] + w[1]), atol=1e-14)
    assert abs(lz[1] - math.log(w[0] + w[1])) < 1e-14
    assert np.allclose(abar[0], a[2]) and abs(lz[0] - 0.5) < 1e-14   # -inf member adds nothing
    assert lz[2] == -np.inf and not np.any(abar[2])                   # empty cluster


# ---------------------------------------------------------------- P12
def check_latent_memory(seed=12):
    """Latent memory of evicted tokens: the feature map against torch's elu, the
    decayed accumulation against its closed form (a weighted matrix product),
    online = one call, empty = identity; the read of a one-token memory returns that
    token's value, a two-token memory the feature-map-weighted average of the
    values; the gate against scipy's expit."""
    r = _rng(seed)
    x = r.standard_normal(50) * 3.0
    ref = torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64)).numpy() + 1.0
    assert np.allclose(OL.phi(x), ref, rtol=0, atol=1e-15), "phi != elu + 1"
    D, n, lam = 6, 9, 0.85
    M0 = r.standard_normal((D, D))
    b0 = np.abs(r.standard_normal(D))
    K = r.standard_normal((n, D))
    V = r.standard_normal((n, D))
    M1, b1 = OL.latent_absorb(M0, b0, K, V, lam)
    w = lam ** (n - 1 - np.arange(n))
    F = torch.nn.functional.elu(torch.tensor(K, dtype=torch.float64)).numpy() + 1.0
    Mref = lam ** n * M0 + (torch.tensor(F * w[:, None]).T @ torch.tensor(V)).numpy()
    bref = lam ** n * b0 + (F * w[:, None]).sum(0)
    assert np.allclose(M1, Mref, rtol=0, atol=1e-12), "decayed accumulation"
    assert np.allclose(b1, bref, rtol=0, atol=1e-12), "stabiliser accumulation"
    Ma, ba = OL.latent_absorb(M0, b0, K[:4], V[:4], lam)
    Mb, bb = OL.latent_absorb(Ma, ba, K[4:], V[4:], lam)
    assert np.allclose(Mb, M1, rtol=0, atol=1e-12) and np.allclose(bb, b1, rtol=0, atol=1e-12)
    Me, be = OL.latent_absorb(M0, b0, K[:0], V[:0], lam)
    assert np.array_equal(Me, M0) and np.array_equal(be, b0), "empty absorb must be identity"
    # one-token memory: the read is that token's value (eps = 0, W_o = I)
    Z = np.zeros((D, D))
    M1t, b1t = OL.latent_absorb(Z, np.zeros(D), K[:1], V[:1], lam)
    q = r.standard_normal(D)
    res, g = OL.latent_read(M1t, b1t, q, np.eye(D), np.zeros(D), 0.0, 0.0)
    assert abs(g - 0.5) < 1e-15 and np.allclose(res, 0.5 * V[0], rtol=0, atol=1e-12)
    # two tokens, lam = 1: weights phi(q).phi(k_i); projection applied after the read
    M2, b2 = OL.latent_absorb(Z, np.zeros(D), K[:2], V[:2], 1.0)
    W = r.standard_normal((D, D))
    fq = torch.nn.functional.elu(torch.tensor(q)).numpy() + 1.0
    a = np.array([fq @ F[0], fq @ F[1]])
    want = W @ ((a[0] * V[0] + a[1] * V[1]) / (a[0] + a[1]))
    wg = r.standard_normal(D)
    res, g = OL.latent_read(M2, b2, q, W, wg, 0.3, 0.0)
    assert abs(g - float(scipy.special.expit(wg @ q + 0.3))) < 1e-15, "gate != sigmoid"
    assert np.allclose(res, g * want, rtol=0, atol=1e-12), "read of a two-token memory"
    o = r.standard_normal(D)
    assert np.allclose(OL.latent_residual(o, M2, b2, q, W, wg, 0.3, 0.0), o + g * want,
                       rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P9
def check_bytes_model():
    """IndexMem's memory-wall estimate: ~320 GB of KV for a 70B model at 1M tokens."""
    per_tok = OB.kv_bytes_per_token(80, 8, 128, 2)
    assert per_tok * (1 << 20) == 320 * (1 << 30)


# ---------------------------------------------------------------- P13
def _sdpa_heads(q, K, V, mask, scale):
    """torch SDPA (float64, CPU) over [B][H] heads of one query each."""
    qt = torch.tensor(q, dtype=torch.float64).unsqueeze(2)          # [B][H][1][D]
    Kt = torch.tensor(K, dtype=torch.float64)                       # [B][H][n][D]
    Vt = torch.tensor(V, dtype=torch.float64)
    mt = torch.tensor(mask, dtype=torch.float64).unsqueeze(2)       # [B][H][1][n]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mt,
                                                         scale=scale)
    return o.squeeze(2).numpy()


def _retention_mask(lb32, pos, t, n, cap):
    """Additive mask of one head: log(beta^d) from the plain power (no product of
    logs), -inf for slots at or beyond the live length."""
    m = np.full(cap, -np.inf)
    for i in range(n):
        d = int(t - pos[i])
        if lb32 is None:
            m[i] = 0.0
            continue
        w = math.exp(float(lb32[i])) ** d                  # beta^0 == 1, also for beta == 0
        m[i] = math.log(w) if w > 0.0 else -np.inf
    return m


def check_decode_attention_gqa(seed=13):
    """Batched grouped-query attention against torch SDPA with K and V repeated per
    group (repeat_interleave: query head h reads KV head h // G), on ragged lengths
    (an empty head included), gapped positions and a distinct decode position per
    sequence.  scale None (or <= 0) must be torch's own default 1/sqrt(D)."""
    r = _rng(seed)
    B, Hkv, G, cap, D = 2, 3, 4, 21, 16
    Hq = Hkv * G
    k = r.standard_normal((B, Hkv, cap, D)) * 1.5
    v = r.standard_normal((B, Hkv, cap, D))
    q = r.standard_normal((B, Hq, D))
    length = np.array([[21, 7, 0], [13, 1, 19]], np.int32)
    pos = np.zeros((B, Hkv, cap), np.int32)
    for b in range(B):
        for g in range(Hkv):
            pos[b, g] = np.sort(r.choice(60, size=cap, replace=False))
    t = np.array([int(pos[0].max()) + 2, int(pos[1].max())], np.int64)
    lb = np.log(r.uniform(0.6, 1.0, size=(B, Hkv, cap))).astype(np.float32)
    # the decode token itself (distance 0) with beta = 0 in one head
    pos[1, 2, length[1, 2] - 1] = t[1]
    lb[1, 2, length[1, 2] - 1] = -np.inf
    for log_beta in (None, lb):
        mask = np.stack([np.stack([_retention_mask(None if log_beta is None else
                                                   log_beta[b, g], pos[b, g], t[b],
                                                   int(length[b, g]), cap)
                                   for g in range(Hkv)]) for b in range(B)])
        Kr = np.repeat(k, G, axis=1)
        Vr = np.repeat(v, G, axis=1)
        Mr = np.repeat(mask, G, axis=1)
        live = np.repeat(length, G, axis=1) > 0
        Mr_safe = np.where(live[:, :, None], Mr, 0.0)        # SDPA of an empty head is NaN
        for scale, torch_scale in ((None, None), (0.0, None), (0.37, 0.37)):
            ref = _sdpa_heads(q, Kr, Vr, Mr_safe, torch_scale)
            sc = 1.0 / math.sqrt(D) if torch_scale is None else torch_scale
            logits = torch.tensor(np.einsum("bhnd,bhd->bhn", Kr, q) * sc + Mr_safe)
            ref_l = torch.logsumexp(logits, dim=-1).numpy()
            out, lse = OT.decode_attention(k, v, log_beta, pos, length, q, t, scale)
            for b in range(B):
                for h in range(Hq):
                    if live[b, h]:
                        assert np.max(np.abs(out[b, h] - ref[b, h])) < 1e-12, \
                            "GQA attention != SDPA with K/V repeated per group"
                        assert abs(lse[b, h] - ref_l[b, h]) < 1e-12, "GQA lse != logsumexp"
                    else:                                  # empty head: (0, -inf)
                        assert not np.any(out[b, h]) and lse[b, h] == -np.inf


# ---------------------------------------------------------------- P14
def _state_sdpa(q, K, V, scale):
    """(out, lse) of one query over a key block: torch SDPA + scipy logsumexp."""
    return _sdpa(q, K, V, scale), float(scipy.special.logsumexp(scale * (K @ q)))


def _asm_batched_case(r, B, Hkv, G, K, D, clustered):
    """A codebook per KV head and queries built so that every answer is known by
    construction: query (b, h) is lambda times entry j(b, h) of KV head h // G (so
    that entry is its cosine argmax), the entries chosen in a group are distinct,
    and the chosen entry's stored state is that same query's attention state over a
    prefix of its own.  The batched lookup + merge must then return j(b, h) and
    attention over [prefix; own tokens] (torch SDPA), i.e. the page's lossless
    merge; any other head map, or looking up with another head's query, picks
    another entry."""
    Hq = Hkv * G
    scale = 1.0 / math.sqrt(D)
    if clustered:
        K1 = K // 3
        u = r.standard_normal((Hkv, K1, D))
        u /= np.linalg.norm(u, axis=2, keepdims=True)
        assign = np.tile(np.repeat(np.arange(K1), 3), (Hkv, 1))
        C = u[np.arange(Hkv)[:, None], assign] + 0.08 * r.standard_normal((Hkv, K, D))
    else:
        C = r.standard_normal((Hkv, K, D)) * r.uniform(0.5, 2.0, size=(Hkv, K, 1))
    abar = r.standard_normal((Hkv, K, D))
    lzb = r.uniform(-2.0, 6.0, size=(Hkv, K))
    q = np.zeros((B, Hq, D))
    want_idx = np.zeros((B, Hq), np.int64)
    want_o = np.zeros((B, Hq, D))
    want_l = np.zeros((B, Hq))
    self_o = np.zeros((B, Hq, D))
    self_l = np.zeros((B, Hq))
    for g in range(Hkv):
        js = r.permutation(K)[: B * G]
        for b in range(B):
            for hh in range(G):
                h = g * G + hh
                j = int(js[b * G + hh])
                want_idx[b, h] = j
                q[b, h] = float(r.uniform(0.5, 3.0)) * C[g, j]
                npre, nself = int(r.integers(1, 9)), int(r.integers(0, 6))
                Kp, Vp = r.standard_normal((npre, D)), r.standard_normal((npre, D))
                Ks, Vs = r.standard_normal((nself, D)), r.standard_normal((nself, D))
                abar[g, j], lzb[g, j] = _state_sdpa(q[b, h], Kp, Vp, scale)
                if nself:
                    self_o[b, h], self_l[b, h] = _state_sdpa(q[b, h], Ks, Vs, scale)
                else:                                       # no own tokens yet
                    self_l[b, h] = -np.inf
                want_o[b, h], want_l[b, h] = _state_sdpa(q[b, h], np.vstack([Kp, Ks]),
                                                         np.vstack([Vp, Vs]), scale)
    return C, abar, lzb, q, self_o, self_l, want_idx, want_o, want_l


def check_asm_batched(seed=14):
    """Batched ASM lookup + merge (linear and two-level) on cases whose index and
    merged output are known by construction (see _asm_batched_case)."""
    r = _rng(seed)
    B, Hkv, G, K, D = 2, 3, 2, 12, 24
    C, abar, lzb, q, so, sl, wi, wo, wl = _asm_batched_case(r, B, Hkv, G, K, D, False)
    out, lse, idx = OA.asm_lookup_merge(q, C, abar, lzb, so, sl)
    assert np.array_equal(idx, wi), "batched lookup: wrong entry (head map / query)"
    assert np.max(np.abs(out - wo)) < 1e-12 and np.max(np.abs(lse - wl)) < 1e-12, \
        "batched lookup + merge != attention over [prefix; own tokens]"
    # two-level: entries near their first-level centroid, stored cluster by cluster
    # (shuffled inside), so the query's own cluster has the best first-level cosine
    C, abar, lzb, q, so, sl, wi, wo, wl = _asm_batched_case(r, B, Hkv, G, K, D, True)
    K1 = K // 3
    c1 = np.stack([np.stack([C[g, 3 * j:3 * j + 3].mean(0) for j in range(K1)])
                   for g in range(Hkv)])
    kid = np.stack([np.concatenate([3 * j + r.permutation(3) for j in range(K1)])
                    for g in range(Hkv)])
    offs = np.tile(np.arange(0, K + 1, 3), (Hkv, 1))
    Cs = np.stack([C[g, kid[g]] for g in range(Hkv)])
    for m in (1, 2, K1):
        out, lse, idx = OA.asm_lookup_merge_hier(q, c1, offs, Cs, kid, m, abar, lzb, so, sl)
        assert np.array_equal(idx, wi), "batched two-level lookup: wrong entry"
        assert np.max(np.abs(out - wo)) < 1e-12 and np.max(np.abs(lse - wl)) < 1e-12, \
            "batched two-level lookup + merge != attention over [prefix; own tokens]"


# ---------------------------------------------------------------- P15
def check_decode_loop_order(seed=15):
    """Two decode steps with budget M = 3 whose evictions are fixed by hand: one token
    with beta = 0.05 goes at step 0, one with beta = 0.5 at step 1 (every other beta
    is 0.95).  Each step's output must be attention over exactly the tokens live
    after the append and before the eviction (torch SDPA over that hand-listed set,
    weights beta^d as plain powers), in the order the TRIM-KV inference section
    gives: the new token joins the cache, is attended to, then the cache is cut back
    to M."""
    r = _rng(seed)
    B, Hkv, G, D, cap, M = 1, 1, 2, 8, 8, 3
    Hq = Hkv * G
    k = np.zeros((B, Hkv, cap, D), np.float32)
    v = np.zeros((B, Hkv, cap, D), np.float32)
    beta = {0: 0.95, 1: 0.05, 2: 0.95, 3: 0.5, 4: 0.95}    # by position
    kr = r.standard_normal((5, D)).astype(np.float32)      # rows by position
    vr = r.standard_normal((5, D)).astype(np.float32)
    lb = np.zeros((B, Hkv, cap), np.float32)
    for p in range(3):
        k[0, 0, p], v[0, 0, p], lb[0, 0, p] = kr[p], vr[p], np.float32(math.log(beta[p]))
    pos = np.zeros((B, Hkv, cap), np.int32)
    pos[0, 0, :3] = [0, 1, 2]
    cache = OE.Cache(k, v, lb, pos, np.array([[3]], np.int32))
    qs = r.standard_normal((2, B, Hq, D))
    k_news = np.stack([kr[3:4][None], kr[4:5][None]])      # [S][B][Hkv][D]
    v_news = np.stack([vr[3:4][None], vr[4:5][None]])
    lb_news = np.array([[[math.log(beta[3])]], [[math.log(beta[4])]]], np.float32)
    final, steps = run_decode(cache, qs, k_news, v_news, lb_news, 3, M)
    live = ([0, 1, 2, 3], [0, 2, 3, 4])                    # attended at steps 0 and 1
    gone = ([1], [3])
    for s in range(2):
        t = 3 + s
        P = np.array(live[s])
        Kl = kr[P].astype(np.float64)
        Vl = vr[P].astype(np.float64)
        # beta as the stored float32 log beta represents it, raised to the distance
        bf = {p: math.exp(float(np.float32(math.log(beta[p])))) for p in P}
        mask = np.array([math.log(bf[p] ** (t - p)) for p in P])
        out, lse, ev, n_ev = steps[s]
        for h in range(Hq):
            ref = _sdpa(qs[s, 0, h], Kl, Vl, 1.0 / math.sqrt(D), mask)
            assert np.max(np.abs(out[0, h] - ref)) < 1e-12, \
                f"step {s}: output is not attention over the appended, un-evicted cache"
            ref_l = scipy.special.logsumexp(Kl @ qs[s, 0, h] / math.sqrt(D) + mask)
            assert abs(lse[0, h] - ref_l) < 1e-12
        assert list(ev[0][0]) == gone[s] and n_ev[0, 0] == 1, f"step {s}: eviction"
    assert final.length[0, 0] == M and list(final.pos[0, 0, :M]) == [0, 2, 4]
    assert np.array_equal(final.k[0, 0, :M], kr[[0, 2, 4]])


# ---------------------------------------------------------------- P16
def _paged_case(r, B, H, n_pages_max, spare_pages=2, max_pages=None):
    """Random paged cache: per head a run of pages with fills 1..32 on distinct
    physical pages, positions ascending along the table with random gaps."""
    D = 4
    max_pages = max_pages or n_pages_max + spare_pages
    phys = n_pages_max + spare_pages + 3
    cap = OE.PAGE * phys
    k = r.integers(0, 1 << 16, size=(B, H, cap, D)).astype(np.uint16)
    v = r.integers(0, 1 << 16, size=(B, H, cap, D)).astype(np.uint16)
    lb = r.uniform(-0.1, 0.0, size=(B, H, cap)).astype(np.float32)
    pos = np.full((B, H, cap), -1, np.int32)
    table = np.full((B, H, max_pages), -7, np.int32)
    fill = np.full((B, H, max_pages), -7, np.int32)
    n_pages = np.zeros((B, H), np.int32)
    length = np.zeros((B, H), np.int32)
    for b in range(B):
        for g in range(H):
            n = int(r.integers(0, n_pages_max + 1))
            perm = r.permutation(phys)[:n]
            p = 0
            for i in range(n):
                f = int(r.integers(1, OE.PAGE + 1))
                for j in range(f):
                    p += int(r.integers(1, 3))
                    pos[b, g, OE.PAGE * perm[i] + j] = p
                table[b, g, i], fill[b, g, i] = perm[i], f
                length[b, g] += f
            n_pages[b, g] = n
    return OE.Cache(k, v, lb, pos, length), OE.Pages(table, fill, n_pages)


def check_paged_erase(seed=16):
    """Block-granular erase: the token sequence it leaves is the contiguous erase's
    (pinned by the set filter above); page by page, written as loops, a page with
    no survivor leaves the table, a page untouched keeps its rows bit for bit, and
    the table keeps its order.  Hand cases fix whole-page drops."""
    r = _rng(seed)
    for _ in range(12):
        c, pg = _paged_case(r, 2, 2, 6)
        top = int(c.pos.max()) + 5
        ranges = []
        for b in range(2):
            edges = np.sort(r.choice(top, size=2 * int(r.integers(0, 5)), replace=False))
            ranges.append(edges.reshape(-1, 2).astype(np.int64))
        c2, pg2, n_er = OE.erase_pages(c, pg, ranges)
        want, n_want = OE.erase_ranges(OE.paged_view(c, pg), ranges)
        got = OE.paged_view(c2, pg2)
        assert np.array_equal(got.length, want.length) and np.array_equal(n_er, n_want)
        assert np.array_equal(c2.length, want.length), "len is not the kept total"
        for b in range(2):
            for g in range(2):
                n = int(want.length[b, g])
                for name in ("k", "v", "pos", "log_beta"):
                    assert np.array_equal(getattr(got, name)[b, g, :n],
                                          getattr(want, name)[b, g, :n]), name
                new_i = 0
                for i in range(int(pg.n_pages[b, g])):
                    p, f = int(pg.table[b, g, i]), int(pg.fill[b, g, i])
                    kept = 0
                    for j in range(f):
                        x = int(c.pos[b, g, 32 * p + j])
                        if not any(s <= x < e for s, e in ranges[b]):
                            kept += 1
                    if kept == 0:
                        continue
                    assert pg2.table[b, g, new_i] == p and pg2.fill[b, g, new_i] == kept
                    if kept == f:
                        assert np.array_equal(c2.k[b, g, 32 * p:32 * p + f],
                                              c.k[b, g, 32 * p:32 * p + f])
                    new_i += 1
                assert pg2.n_pages[b, g] == new_i
    # hand case: pages 3 (positions 0..31) and 1 (32..40); erasing [32, 41) drops
    # page 1, erasing [0, 32) drops page 3, erasing [30, 34) keeps both, partly
    pos = np.zeros((1, 1, 128), np.int32)
    pos[0, 0, 96:128] = np.arange(32)
    pos[0, 0, 32:41] = np.arange(32, 41)
    k = np.arange(128 * 2, dtype=np.uint16).reshape(1, 1, 128, 2)
    c = OE.Cache(k, k.copy(), None, pos, np.array([[41]], np.int32))
    pg = OE.Pages(np.array([[[3, 1]]], np.int32), np.array([[[32, 9]]], np.int32),
                  np.array([[2]], np.int32))
    for rg, tab, fil in (([[32, 41]], [3], [32]), ([[0, 32]], [1], [9]),
                         ([[30, 34]], [3, 1], [30, 7])):
        c2, pg2, n_er = OE.erase_pages(c, pg, [np.array(rg)])
        n = int(pg2.n_pages[0, 0])
        assert list(pg2.table[0, 0, :n]) == tab and list(pg2.fill[0, 0, :n]) == fil, rg
        assert n_er[0, 0] == 41 - sum(fil)
    c2, pg2, _ = OE.erase_pages(c, pg, [np.array([[30, 34]])])
    assert list(c2.pos[0, 0, 32:39]) == list(range(34, 41))
    assert np.array_equal(c2.k[0, 0, 32:39], k[0, 0, 34:41])


def check_paged_append(seed=17):
    """Decode token of a paged cache: into the last page's next slot while it has
    one, else onto the free page given (added to the table), else not stored."""
    pos = np.zeros((1, 2, 96), np.int32)
    k = np.zeros((1, 2, 96, 2), np.uint16)
    c = OE.Cache(k, k.copy(), None, pos, np.array([[5, 32]], np.int32))
    pg = OE.Pages(np.array([[[2, -1], [0, -1]]], np.int32),
                  np.array([[[5, 0], [32, 0]]], np.int32), np.array([[1, 1]], np.int32))
    kn = np.array([[[7, 7], [9, 9]]], np.uint16)
    st = OE.paged_append(c, pg, kn, kn, None, np.array([50]), np.array([[1, 1]]))
    assert st.tolist() == [[True, True]]
    assert c.pos[0, 0, 64 + 5] == 50 and list(c.k[0, 0, 69]) == [7, 7]
    assert pg.fill[0, 0, 0] == 6 and pg.n_pages[0, 0] == 1, "free page taken while room"
    assert pg.table[0, 1, 1] == 1 and pg.fill[0, 1, 1] == 1 and pg.n_pages[0, 1] == 2
    assert c.pos[0, 1, 32] == 50 and list(c.k[0, 1, 32]) == [9, 9]
    assert c.length.tolist() == [[6, 33]]
    # no room: a full last page, no free page (or a full table)
    pg2 = OE.Pages(np.array([[[0, 1], [0, 1]]], np.int32),
                   np.array([[[32, 32], [32, 0]]], np.int32), np.array([[2, 1]], np.int32))
    st = OE.paged_append(c, pg2, kn, kn, None, np.array([51]), np.array([[2, -1]]))
    assert st.tolist() == [[False, False]] and c.length.tolist() == [[6, 33]]
    # the view walks the table: pages [2, 0] with fills [3, 2] are slots 64-66, 0-1
    pg3 = OE.Pages(np.array([[[2, 0], [0, 0]]], np.int32),
                   np.array([[[3, 2], [1, 0]]], np.int32), np.array([[2, 1]], np.int32))
    assert list(OE.paged_slots(pg3, 0, 0)) == [64, 65, 66, 0, 1]


def run_decode(*a, **kw):
    import oracle.decode as OD
    return OD.run_decode_steps(*a, **kw)


ALL = [check_attention_library, check_bias_closed_form, check_split_merge,
       check_asm_lossless, check_evict_bruteforce, check_evict_sliding_window,
       check_evict_invariants, check_compaction, check_erase_bruteforce,
       check_lookup_bruteforce, check_hier_lookup, check_asm_build, check_latent_memory, check_bytes_model,
       check_decode_attention_gqa, check_asm_batched, check_decode_loop_order,
       check_paged_erase, check_paged_append]
