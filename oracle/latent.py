"""Float64 latent memory of evicted tokens (residual read-out).

TEST INFRASTRUCTURE ONLY (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

"IndexMem: Learned KV-Cache Eviction with Latent Memory for Long-Context LLM
Inference", technical summary, section 2 (methodology), part B (latent memory for
evicted tokens): every evicted token updates, online, a fixed-size state matrix M
and a stabiliser vector b by an outer-product accumulation with decay (fast
weights); a projection and a gate g(q) (slow weights, trained) read the memory,
and the attention output becomes o = o_attn + g(q) * m(q), o_attn being attention
over the kept tokens.

Readings (the page names the parts, not their formulas; the trained parts are
replaced by constants the caller supplies):
* one state per KV head: M [D][D], b [D], starting at zero;
* feature map phi(x) = elu(x) + 1 (positive, so the read's normaliser is > 0);
* absorbing an evicted token (k, v): M <- lam * M + phi(k) v^T, b <- lam * b + phi(k),
  one decay step per token, tokens taken in slot (= position) order;
* read for a query q: r = M^T phi(q) / (b . phi(q) + eps) (the stabiliser
  normalises the read), m(q) = W_o r (projection), g(q) = sigmoid(w_g . q + c_g)
  (per query head), o = o_attn + g(q) m(q).
"""
from __future__ import annotations

import numpy as np


def phi(x):
    """elu(x) + 1."""
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def latent_absorb(Mst, bst, K_ev, V_ev, lam):
    """State after absorbing the evicted rows K_ev, V_ev [n][D] in order."""
    Mst = np.array(Mst, np.float64)
    bst = np.array(bst, np.float64)
    for k, v in zip(np.asarray(K_ev, np.float64), np.asarray(V_ev, np.float64)):
        f = phi(k)
        Mst = lam * Mst + np.outer(f, v)
        bst = lam * bst + f
    return Mst, bst


def latent_read(Mst, bst, q, W_o, w_g, c_g, eps):
    """(g(q) * m(q), g(q)) for one query head."""
    f = phi(q)
    r = (np.asarray(Mst, np.float64).T @ f) / (float(np.asarray(bst, np.float64) @ f) + eps)
    m = np.asarray(W_o, np.float64) @ r
    g = 1.0 / (1.0 + np.exp(-(float(np.asarray(w_g, np.float64) @ np.asarray(q, np.float64))
                              + float(c_g))))
    return g * m, g


def latent_residual(o_attn, Mst, bst, q, W_o, w_g, c_g, eps):
    """o = o_attn + g(q) m(q)."""
    res, _ = latent_read(Mst, bst, q, W_o, w_g, c_g, eps)
    return np.asarray(o_attn, np.float64) + res
