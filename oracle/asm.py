"""Float64 Attention-State Memory lookup (linear and hierarchical) and merge.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

Context Memorization, method steps, step 3: a decode query looks up the
centroid with the largest cosine similarity and fetches its stored state
(abar, Zbar); step 4 merges that state with the query's own attention state
(a, Z) over the generated tokens, weighting each by its normaliser.  The GQA
extension (technical-novelty section) keeps centroids per KV head; here every
query head looks up with its own query in its KV head's codebook.  The same
section's hierarchical index replaces the linear scan by two levels: the query
is first compared with first-level centroids, and only the entries of the
best-scoring first-level clusters are compared exactly (the experiments expand
the top 16 first-level centroids and match the linear lookup's top-1).
"""
from __future__ import annotations

import numpy as np

from .attn import merge_states, state_to_out_lse

NEG_INF = -np.inf


def cosine_similarities(q, centroids):
    """cos(q, c_k) = (q . c_k) / (|q| |c_k|) for every centroid, in float64.

    The stored centroid values are used as they are (not re-normalised).  A zero
    query or a zero centroid has no defined cosine; it is taken as -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    C = np.asarray(centroids, dtype=np.float64)
    qn = np.sqrt(np.sum(q * q))
    cn = np.sqrt(np.sum(C * C, axis=1))
    with np.errstate(invalid="ignore", divide="ignore"):
        cos = (C @ q) / (cn * qn)
    bad = (cn == 0.0) | (qn == 0.0)
    return np.where(bad, NEG_INF, cos)


def cosine_lookup(q, centroids):
    """argmax_k cos(q, c_k); equal similarities go to the lowest k."""
    cos = cosine_similarities(q, centroids)
    return int(np.argmax(cos))           # first maximum


def hier_lookup(q, c1, offs, centroids, kid, m):
    """Two-level cosine lookup; returns an original entry index.

    c1 [K1][D]: first-level centroids.  The entries of first-level cluster j sit
    at positions offs[j] .. offs[j+1]-1 of ``centroids`` (stored cluster by
    cluster); kid[p] is the original index of the entry at position p.
    1. cos(q, c1_j) for every j; keep the m largest (equal similarities: the
       lower j first).
    2. Among the entries of the kept clusters, the largest cos(q, c); equal
       similarities go to the lowest original index.
    A zero query, or kept clusters without entries, give index 0 (as the linear
    lookup gives 0 for a zero query).
    """
    q = np.asarray(q, dtype=np.float64)
    if not np.any(q != 0.0):
        return 0
    K1 = len(c1)
    s1 = cosine_similarities(q, c1)
    order = np.lexsort((np.arange(K1), -s1))      # descending similarity, then j
    kept = order[:m]
    pos = np.concatenate([np.arange(offs[j], offs[j + 1]) for j in kept]).astype(np.int64)
    if pos.size == 0:
        return 0
    s = cosine_similarities(q, np.asarray(centroids)[pos])
    ids = np.asarray(kid)[pos]
    best = np.lexsort((ids, -s))[0]                # descending similarity, then index
    return int(ids[best])


def asm_merge(out, lse, abar, log_zbar):
    """Merge a query's own (out, lse) with a stored state (abar, log Zbar).

    out' = Z/(Z+Zbar) * out + Zbar/(Z+Zbar) * abar, lse' = log(Z + Zbar), with
    Z = exp(lse).  lse = -inf (no own tokens) gives the stored state unchanged.
    """
    own = (np.asarray(out, np.float64), float(lse), 1.0) if lse != NEG_INF else \
        (np.zeros(len(out)), NEG_INF, 0.0)
    mem = (np.asarray(abar, np.float64), float(log_zbar), 1.0) if log_zbar != NEG_INF else \
        (np.zeros(len(out)), NEG_INF, 0.0)
    return state_to_out_lse(merge_states([own, mem]))


def asm_lookup_merge(q, centroids, abar, log_zbar, self_out, self_lse):
    """Batched lookup + merge.

    q [B][Hq][D]; centroids, abar [Hkv][K][D]; log_zbar [Hkv][K];
    self_out [B][Hq][D]; self_lse [B][Hq].  Query head h uses KV head floor(h/G).
    Returns (out [B][Hq][D], lse [B][Hq], idx [B][Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = centroids.shape[0]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    idx = np.zeros((B, Hq), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            c = cosine_lookup(q[b, h], centroids[g])
            idx[b, h] = c
            out[b, h], lse[b, h] = asm_merge(self_out[b, h], self_lse[b, h],
                                             abar[g][c], log_zbar[g][c])
    return out, lse, idx


def asm_lookup_merge_hier(q, c1, offs, centroids, kid, m, abar, log_zbar, self_out, self_lse):
    """Batched hierarchical lookup + merge.

    q [B][Hq][D]; c1 [Hkv][K1][D]; offs [Hkv][K1+1]; centroids [Hkv][K][D] in
    cluster order with kid [Hkv][K] their original indices; abar [Hkv][K][D] and
    log_zbar [Hkv][K] in original index order.  Returns (out, lse, idx).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = c1.shape[0]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    idx = np.zeros((B, Hq), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            c = hier_lookup(q[b, h], c1[g], offs[g], centroids[g], kid[g], m)
            idx[b, h] = c
            out[b, h], lse[b, h] = asm_merge(self_out[b, h], self_lse[b, h],
                                             abar[g][c], log_zbar[g][c])
    return out, lse, idx
