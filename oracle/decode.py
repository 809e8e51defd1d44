"""Float64 decode loop: append, attend, evict -- one step after another.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Cache What Lasts" section 2.2 (inference): each generated token gets its
retention score when it is produced, joins the cache, and when the cache then
holds more than M tokens the lowest-scoring ones are evicted.  The order within
a step is taken as: append the new token, attend over every live token
(including the new one), then evict to M and compact.
"""
from __future__ import annotations

import numpy as np

from .attn import decode_attention
from .evict import append_tokens, evict_to_budget


def run_decode_steps(cache, qs, k_news, v_news, lb_news, t0, M, scale=None):
    """Run len(qs) decode steps on a copy of ``cache``.

    qs [S][B][Hq][D] float64 values; k_news, v_news [S][B][Hkv][D] in the cache's
    storage dtype; lb_news [S][B][Hkv] float32 or None; token positions t0 + s.
    Returns (final cache, per-step list of (out, lse, evicted_pos, n_evicted)).
    """
    c = cache.copy()
    B = c.length.shape[0]
    steps = []
    for s in range(len(qs)):
        t = np.full(B, t0 + s, dtype=np.int64)
        append_tokens(c, k_news[s], v_news[s], None if lb_news is None else lb_news[s], t)
        k = c.values("k")
        v = c.values("v")
        out, lse = decode_attention(k, v, c.log_beta, c.pos, c.length, qs[s], t, scale)
        c, ev, n_ev = evict_to_budget(c, t, M)
        steps.append((out, lse, ev, n_ev))
    return c, steps
