"""Float64 construction of an Attention-State Memory (offline calibration).

TEST INFRASTRUCTURE ONLY (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

"Context Memorization for Efficient Long Context Generation", method steps:
step 1 (collection) -- every calibration query q (a query of a response trajectory
run after the prefix) gets its attention state over the prefix,
a_p(q) = attn(q, K_p, V_p) and Z_p(q) = sum_k exp(q.k / sqrt(d_h)); the core-method
section adds that the prefix may be encoded in chunks whose states are merged (the
online-softmax identity makes this lossless).  Step 2 (clustering) -- K-means over
the collected query vectors gives K clusters; a cluster's query centroid is the
mean of its queries and its state the merge of its members' states (the page's
attention-aware aggregation, as opposed to a plain average).

Readings (where the page is silent): Euclidean K-means run as a fixed number of
Lloyd iterations from given initial centroids; each iteration assigns every query
to its nearest centroid (ties to the lower index) and moves every centroid to the
mean of its members, a centroid without members staying where it is; the memory
uses the last assignment.  Chunks are equal consecutive slices of the prefix
(the last may be shorter).  A cluster without members stores the empty state.
"""
from __future__ import annotations

import numpy as np

from .attn import attention_state, merge_states, state_to_out_lse

NEG_INF = -np.inf


def chunk_bounds(L, chunks):
    """Consecutive slices of a length-L prefix: ceil(L / chunks) tokens each."""
    size = -(-L // max(int(chunks), 1)) if L else 0
    return [(c0, min(L, c0 + size)) for c0 in range(0, L, size)] if size else []


def prefix_states(Q, K, V, scale, chunks=1):
    """(a [N][D], lse [N]): each query's attention state over the prefix (K, V),
    computed chunk by chunk and merged.  lse = log of the page's Z (= m + log Z')."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, D = Q.shape
    a = np.zeros((N, D))
    lse = np.full(N, NEG_INF)
    bounds = chunk_bounds(K.shape[0], chunks)
    for i in range(N):
        parts = [attention_state(Q[i], K[c0:c1], V[c0:c1], np.zeros(c1 - c0), scale)
                 for (c0, c1) in bounds]
        a[i], lse[i] = state_to_out_lse(merge_states(parts))
    return a, lse


def nearest_centroid(x, C):
    """Index of the centroid nearest to x in Euclidean distance (ties: lower index)."""
    d2 = np.sum((np.asarray(C, np.float64) - np.asarray(x, np.float64)) ** 2, axis=1)
    return int(np.argmin(d2))


def centroid_update(X, assign, C):
    """Mean of each cluster's members; a centroid without members keeps its place."""
    X = np.asarray(X, np.float64)
    C = np.array(C, np.float64)
    for k in range(C.shape[0]):
        members = X[assign == k]
        if members.shape[0]:
            C[k] = members.mean(axis=0)
    return C


def kmeans(X, init, iters):
    """Lloyd iterations; returns (assignment of the last iteration, centroids)."""
    X = np.asarray(X, np.float64)
    C = np.array(init, np.float64)
    assign = np.zeros(X.shape[0], np.int64)
    for _ in range(iters):
        assign = np.array([nearest_centroid(x, C) for x in X], np.int64)
        C = centroid_update(X, assign, C)
    return assign, C


def aggregate_states(assign, a, lse, K):
    """Per cluster: the merge of its members' states (members in index order).
    Returns (abar [K][D], log_zbar [K]); an empty cluster gives (0, -inf)."""
    a = np.asarray(a, np.float64)
    D = a.shape[1]
    abar = np.zeros((K, D))
    lz = np.full(K, NEG_INF)
    for k in range(K):
        idx = np.nonzero(np.asarray(assign) == k)[0]
        states = [(a[i], float(lse[i]), 1.0) if lse[i] != NEG_INF else (np.zeros(D), NEG_INF, 0.0)
                  for i in idx]
        abar[k], lz[k] = state_to_out_lse(merge_states(states)) if states else (np.zeros(D),
                                                                                 NEG_INF)
    return abar, lz


def build_memory(Q, Kp, Vp, scale, chunks, init, iters):
    """Steps 1 and 2 for one KV head: (centroids, abar, log_zbar, assignment)."""
    a, lse = prefix_states(Q, Kp, Vp, scale, chunks)
    assign, C = kmeans(Q, init, iters)
    abar, lz = aggregate_states(assign, a, lse, np.asarray(init).shape[0])
    return C, abar, lz, assign
