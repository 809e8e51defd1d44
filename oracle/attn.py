"""Float64 retention-biased decode attention and the attention-state merge.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

State convention.  The Context Memorization page stores an attention state as
(a, Z): a is the normalised attention output over a key block and Z the sum of
exp(q.k/sqrt(d)) over that block.  Z overflows any fixed-width float for large
logits, so the state is carried here as (a, m, Z) with Z = sum exp(s - m); the
page's normaliser is exp(m) * Z.  The empty state is (0, -inf, 0).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def retention_bias(log_beta, pos, t):
    """Additive logit bias (t - i) * log(beta_i) of every token.

    "Cache What Lasts" section 2.1 (retention-gated attention): token i's weight
    at step t is scaled by beta_i^(t-i), i.e. exp(q.k + (t-i) log beta_i).
    Readings: i is the token's absolute position (not its slot); the bias is 0 at
    distance 0 because beta^0 = 1, even when log beta = -inf; with no retention
    array (log_beta is None) beta == 1 and the bias is 0.
    """
    pos = np.asarray(pos, dtype=np.int64)
    if log_beta is None:
        return np.zeros(pos.shape, dtype=np.float64)
    dist = (np.int64(t) - pos).astype(np.float64)
    lb = np.asarray(log_beta, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        bias = dist * lb
    return np.where(dist == 0.0, 0.0, bias)


def attention_state(q, K, V, bias, scale):
    """Attention state (a, m, Z) of one query over one key block.

    Logits s_i = scale * (q . k_i) + bias_i (the dot product is scaled, the
    retention bias is not).  m = max_i s_i, Z = sum_i exp(s_i - m),
    a = sum_i exp(s_i - m) v_i / Z.  An empty block, or one in which every weight
    is zero (all logits -inf), gives the empty state (0, -inf, 0).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    D = V.shape[-1]
    if K.shape[0] == 0:
        return np.zeros(D), NEG_INF, 0.0
    s = scale * (K @ q) + np.asarray(bias, dtype=np.float64)
    m = float(np.max(s))
    if m == NEG_INF:
        return np.zeros(D), NEG_INF, 0.0
    w = np.exp(s - m)
    Z = float(np.sum(w))
    a = (w @ V) / Z
    return a, m, Z


def merge_states(states):
    """Fold attention states left to right with the merge operator.

    Context Memorization, method steps, step 2: merging (a_A, Z_A) and (a_B, Z_B)
    gives ((Z_A a_A + Z_B a_B) / (Z_A + Z_B), Z_A + Z_B).  With Z = exp(m) * Z',
    both normalisers are brought to the common reference max(m_A, m_B) first.
    The empty state (0, -inf, 0) is the identity.
    """
    a, m, Z = None, NEG_INF, 0.0
    for a2, m2, Z2 in states:
        a2 = np.asarray(a2, dtype=np.float64)
        if Z2 == 0.0:
            if a is None:
                a = np.zeros_like(a2)
            continue
        if Z == 0.0:
            a, m, Z = a2.copy(), float(m2), float(Z2)
            continue
        M = max(m, float(m2))
        wa = Z * np.exp(m - M)
        wb = Z2 * np.exp(float(m2) - M)
        a = (wa * a + wb * a2) / (wa + wb)
        m, Z = M, wa + wb
    return a, m, Z


def state_to_out_lse(state):
    """Output vector and log normaliser (log-sum-exp of the logits) of a state."""
    a, m, Z = state
    if Z == 0.0:
        return np.zeros_like(a), NEG_INF
    return a, m + float(np.log(Z))


def attention(q, K, V, log_beta, pos, t, scale):
    """Decode attention of one query over one head's live tokens -> (out, lse)."""
    bias = retention_bias(log_beta, pos, t)
    return state_to_out_lse(attention_state(q, K, V, bias, scale))


def split_attention(q, K, V, log_beta, pos, t, scale, bounds):
    """Split-K form: one state per token block [bounds[j], bounds[j+1]), then merge.

    The online-softmax identity (Context Memorization, background knowledge)
    says the merged result equals attention over all keys for any partition.
    Returns (out, lse, partial_states).
    """
    bias = retention_bias(log_beta, pos, t)
    parts = []
    for j in range(len(bounds) - 1):
        lo, hi = bounds[j], bounds[j + 1]
        parts.append(attention_state(q, K[lo:hi], V[lo:hi], bias[lo:hi], scale))
    out, lse = state_to_out_lse(merge_states(parts))
    return out, lse, parts


def decode_attention(k, v, log_beta, pos, length, q, t, scale=None):
    """Grouped-query decode attention over a whole cache.

    k, v [B][Hkv][cap][D]; log_beta [B][Hkv][cap] or None; pos [B][Hkv][cap];
    length [B][Hkv]; q [B][Hq][D]; t [B].  Query head h reads KV head
    floor(h / G) with G = Hq / Hkv (contiguous groups: the pages say query heads
    share KV heads under GQA but not which; this is the usual grouping).
    scale defaults to 1/sqrt(D).  Returns out [B][Hq][D], lse [B][Hq] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            n = int(length[b][g])
            lb = None if log_beta is None else log_beta[b][g][:n]
            out[b, h], lse[b, h] = attention(q[b, h], k[b][g][:n], v[b][g][:n], lb,
                                             pos[b][g][:n], int(t[b]), scale)
    return out, lse
