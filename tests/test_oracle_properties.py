"""Property-based pins of the oracle (hypothesis, CPU).

Random small shapes, with values drawn from small sets so that ties, zero and
infinite log betas, distance 0 and empty heads come up often.  Each property states
what the pages fix in a form that shares no arithmetic with the oracle:

* attention with the retention bias: weights exp(scale q.k_i) * beta_i^(t-i) with
  beta_i^(t-i) an integer power of beta_i (no logarithms), normalised
  ("Cache What Lasts" section 2.1);
* split and merge: any partition of the keys into blocks, merged in any order,
  gives the same output and log-normaliser as one pass (Context Memorization,
  background: the online-softmax identity; method step 2: the merge operator);
* eviction: the kept set is the M tokens with the largest exact retention score,
  compared as exact rationals (the float32 log beta times the integer distance,
  as a Fraction), ties kept by the higher position ("Cache What Lasts" section
  2.2, inference);
* erasure: a plain set filter of the positions (MEMENTO, blocks and compression);
* compaction: the kept rows, in slot order, bit for bit.
"""
from fractions import Fraction

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=150, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])

BETAS = [1.0, 0.5, 0.25, 0.9, 0.75, 0.0]   # exact binary fractions and 0.9, 0.75, 0


@st.composite
def head(draw, max_n=10, D=None):
    n = draw(st.integers(0, max_n))
    D = D or draw(st.integers(1, 5))
    gaps = draw(st.lists(st.integers(1, 4), min_size=n, max_size=n))
    pos = np.cumsum([0] + gaps)[1:].astype(np.int64) if n else np.zeros(0, np.int64)
    t = int(pos[-1]) + draw(st.integers(0, 3)) if n else draw(st.integers(0, 5))
    beta = np.array([draw(st.sampled_from(BETAS)) for _ in range(n)], np.float64)
    rng = np.random.default_rng(draw(st.integers(0, 2 ** 31)))
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    return n, D, pos, t, beta, q, K, V


def _log_beta(beta):
    with np.errstate(divide="ignore"):
        return np.log(beta).astype(np.float32)


@SETTINGS
@given(head(), st.sampled_from([1.0, 0.5, 0.125]))
def test_attention_is_the_power_weighted_average(h, scale):
    n, D, pos, t, beta, q, K, V = h
    lb = _log_beta(beta)
    out, lse = oracle.attention(q, K, V, lb, pos, t, scale)
    # weights with beta_i^(t - i) as an integer power of the float32 beta the
    # oracle sees (exp of its log), 0 ** 0 = 1 at distance 0
    b32 = np.exp(lb.astype(np.float64))
    w = np.array([np.exp(scale * float(q @ K[i])) * b32[i] ** int(t - pos[i]) for i in range(n)])
    if n == 0 or w.sum() == 0.0:
        assert lse == -np.inf and np.all(out == 0.0)
        return
    ref = (w[:, None] * V).sum(0) / w.sum()
    assert np.allclose(out, ref, rtol=1e-9, atol=1e-12)
    assert np.isclose(lse, np.log(w.sum()), rtol=1e-9, atol=1e-9)


@SETTINGS
@given(head(max_n=14), st.data())
def test_split_and_merge_in_any_order_equals_one_pass(h, data):
    n, D, pos, t, beta, q, K, V = h
    lb = _log_beta(beta)
    cuts = sorted(data.draw(st.lists(st.integers(0, n), max_size=5)))
    bounds = [0] + cuts + [n]
    blocks = [(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1)]
    bias = oracle.retention_bias(lb, pos, t)
    states = [oracle.attention_state(q, K[s:e], V[s:e], bias[s:e], 0.5) for s, e in blocks]
    perm = data.draw(st.permutations(range(len(states))))
    got = oracle.state_to_out_lse(oracle.merge_states([states[i] for i in perm]))
    ref = oracle.attention(q, K, V, lb, pos, t, 0.5)
    assert np.allclose(got[0], ref[0], rtol=1e-9, atol=1e-12)
    assert (got[1] == ref[1] == -np.inf) or np.isclose(got[1], ref[1], rtol=1e-12, atol=1e-12)


def _exact_score(lb32, d):
    """Exact log of beta^d as a sortable value: -inf, or the rational d * log beta."""
    if d == 0:
        return (1, Fraction(0))
    if np.isneginf(lb32):
        return (0, Fraction(0))
    return (1, Fraction(float(lb32)) * d)


@SETTINGS
@given(head(max_n=12, D=1), st.data())
def test_eviction_keeps_the_exact_top_m(h, data):
    n, _, pos, t, beta, *_ = h
    M = data.draw(st.integers(0, n + 1))
    lb = _log_beta(beta)
    keep, gone = oracle.evict_plan(lb, pos, n, t, M)
    if n <= M:
        assert keep.all() and gone.size == 0
        return
    ranked = sorted(range(n), key=lambda i: (_exact_score(lb[i], int(t - pos[i])), int(pos[i])))
    want_gone = set(ranked[: n - M])
    assert set(np.nonzero(~keep)[0].tolist()) == want_gone
    assert gone.tolist() == sorted(int(pos[i]) for i in want_gone)


@SETTINGS
@given(st.lists(st.integers(0, 60), min_size=0, max_size=25, unique=True),
       st.lists(st.integers(-5, 70), min_size=0, max_size=10, unique=True))
def test_erasure_is_a_set_filter(positions, edges):
    pos = np.array(sorted(positions), np.int64)
    e = sorted(edges)[: len(edges) // 2 * 2]
    ranges = np.array(e, np.int64).reshape(-1, 2)
    keep = oracle.erase_plan(pos, pos.size, ranges)
    erased = set()
    for s, f in ranges.tolist():
        erased |= set(range(s, f))
    assert keep.tolist() == [int(p) not in erased for p in pos]


@SETTINGS
@given(st.integers(1, 12), st.integers(1, 4), st.data())
def test_compaction_keeps_rows_in_slot_order(n, D, data):
    rng = np.random.default_rng(data.draw(st.integers(0, 2 ** 31)))
    cap = n + 2
    k = rng.integers(0, 1 << 16, (1, 1, cap, D)).astype(np.uint16)
    v = rng.integers(0, 1 << 16, (1, 1, cap, D)).astype(np.uint16)
    lb = -rng.random((1, 1, cap)).astype(np.float32)
    pos = np.arange(cap, dtype=np.int32).reshape(1, 1, cap) * 3
    c = oracle.Cache(k.copy(), v.copy(), lb.copy(), pos.copy(), np.array([[n]], np.int32))
    keep = np.array(data.draw(st.lists(st.booleans(), min_size=n, max_size=n)))
    kept = oracle.compact_unit(c, 0, 0, keep)
    idx = [i for i in range(n) if keep[i]]
    assert kept == len(idx) == c.length[0, 0]
    for name, orig in (("k", k), ("v", v), ("log_beta", lb), ("pos", pos)):
        got = getattr(c, name)[0, 0, :kept]
        assert np.array_equal(got.view(np.uint8), orig[0, 0, idx].view(np.uint8)), name
