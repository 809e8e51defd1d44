"""Planted mistakes in the oracle (on the CPU) must each fail a pin.

Every mutant below is a plausible slip -- a dropped term, a wrong sign or
index, a transposed operand, a reversed tie-break -- patched into the oracle
module for the duration of one test.  The test passes only if at least one pin
raises, which shows the pins can tell a wrong oracle from a right one.
"""
import numpy as np
import pytest

import oracle.asm as OA
import oracle.asm_build as OAB
import oracle.attn as OT
import oracle.decode as OD
import oracle.evict as OE
import oracle.latent as OL
import pins

_orig_bias = OT.retention_bias
_orig_state = OT.attention_state
_orig_merge = OT.merge_states
_orig_keys = OE.retention_keys
_orig_plan = OE.evict_plan
_orig_hier = OA.hier_lookup
_orig_update = OAB.centroid_update
_orig_bounds = OAB.chunk_bounds
_orig_absorb = OL.latent_absorb
_orig_read = OL.latent_read
_orig_lookup = OA.cosine_lookup
_orig_hier_b = OA.hier_lookup


def bias_sign_flipped(log_beta, pos, t):
    return -_orig_bias(log_beta, pos, t)


def bias_dropped(log_beta, pos, t):
    return _orig_bias(None, pos, t)


def bias_uses_slot(log_beta, pos, t):
    slots = np.arange(np.asarray(pos).shape[0]) + (int(t) - int(np.asarray(pos)[-1]) if
                                                   np.asarray(pos).size else 0)
    return _orig_bias(log_beta, slots, t)


def bias_ignores_zero_distance(log_beta, pos, t):
    pos = np.asarray(pos, dtype=np.int64)
    if log_beta is None:
        return np.zeros(pos.shape)
    with np.errstate(invalid="ignore"):
        return (t - pos).astype(np.float64) * np.asarray(log_beta, np.float64)


def state_bias_scaled(q, K, V, bias, scale):
    return _orig_state(q, K, V, np.asarray(bias) * scale, scale)


def state_no_scale(q, K, V, bias, scale):
    return _orig_state(q, K, V, bias, 1.0)


def state_k_for_v(q, K, V, bias, scale):
    return _orig_state(q, K, K, bias, scale)


def merge_weights_swapped(states):
    a, m, Z = None, -np.inf, 0.0
    for a2, m2, Z2 in states:
        a2 = np.asarray(a2, dtype=np.float64)
        if Z2 == 0.0:
            a = np.zeros_like(a2) if a is None else a
            continue
        if Z == 0.0:
            a, m, Z = a2.copy(), float(m2), float(Z2)
            continue
        M = max(m, float(m2))
        wa, wb = Z * np.exp(m - M), Z2 * np.exp(float(m2) - M)
        a = (wb * a + wa * a2) / (wa + wb)
        m, Z = M, wa + wb
    return a, m, Z


def merge_no_rescale(states):
    a, m, Z = None, -np.inf, 0.0
    for a2, m2, Z2 in states:
        a2 = np.asarray(a2, dtype=np.float64)
        if Z2 == 0.0:
            a = np.zeros_like(a2) if a is None else a
            continue
        if Z == 0.0:
            a, m, Z = a2.copy(), float(m2), float(Z2)
            continue
        a = (Z * a + Z2 * a2) / (Z + Z2)
        m, Z = max(m, float(m2)), Z + Z2
    return a, m, Z


def keys_negated(log_beta, pos, t):
    return -_orig_keys(log_beta, pos, t)


def keys_no_distance(log_beta, pos, t):
    pos = np.asarray(pos)
    if log_beta is None:
        return np.zeros(pos.shape)
    return np.asarray(log_beta, np.float64) + 0.0


def plan_ties_high_first(log_beta, pos, n, t, M):
    keep = np.ones(n, dtype=bool)
    if n <= M:
        return keep, np.zeros(0, np.int32)
    p = np.asarray(pos)[:n].astype(np.int64)
    lb = None if log_beta is None else np.asarray(log_beta)[:n]
    key = OE.retention_keys(lb, p, t)
    order = np.lexsort((-p, key))
    keep[order[: n - M]] = False
    return keep, np.sort(p[~keep]).astype(np.int32)


def plan_off_by_one(log_beta, pos, n, t, M):
    return _orig_plan(log_beta, pos, n, t, M + 1)


def erase_closed(pos, n, ranges):
    p = np.asarray(pos)[:n].astype(np.int64)
    keep = np.ones(n, dtype=bool)
    for s, e in np.asarray(ranges, dtype=np.int64).reshape(-1, 2):
        keep &= ~((p >= s) & (p <= e))
    return keep


def lookup_raw_dot(q, centroids):
    return int(np.argmax(np.asarray(centroids, np.float64) @ np.asarray(q, np.float64)))


def lookup_last_tie(q, centroids):
    cos = OA.cosine_similarities(q, centroids)
    return int(len(cos) - 1 - np.argmax(cos[::-1]))


def asm_merge_linear(out, lse, abar, log_zbar):
    w1, w2 = lse, log_zbar
    if not np.isfinite(w1):
        return np.asarray(abar, np.float64), log_zbar
    if not np.isfinite(w2):
        return np.asarray(out, np.float64), lse
    return (w1 * np.asarray(out) + w2 * np.asarray(abar)) / (w1 + w2), np.logaddexp(lse, log_zbar)


def _hier(q, c1, offs, centroids, kid, m, first_dot=False, keep=None, high_j=False,
          pos_out=False, tie_pos=False):
    q = np.asarray(q, np.float64)
    if not np.any(q != 0.0):
        return 0
    K1 = len(c1)
    s1 = np.asarray(c1, np.float64) @ q if first_dot else OA.cosine_similarities(q, c1)
    order = np.lexsort((-np.arange(K1) if high_j else np.arange(K1), -s1))
    kept = order[:m if keep is None else keep]
    pos = np.concatenate([np.arange(offs[j], offs[j + 1]) for j in kept] +
                         [np.zeros(0, np.int64)]).astype(np.int64)
    if pos.size == 0:
        return 0
    s = OA.cosine_similarities(q, np.asarray(centroids)[pos])
    ids = np.asarray(kid)[pos]
    best = np.lexsort((pos if tie_pos else ids, -s))[0]
    return int(pos[best]) if pos_out else int(ids[best])


def hier_first_level_dot(q, c1, offs, centroids, kid, m):
    return _hier(q, c1, offs, centroids, kid, m, first_dot=True)


def hier_keeps_one_fewer(q, c1, offs, centroids, kid, m):
    return _hier(q, c1, offs, centroids, kid, m, keep=max(m - 1, 0))


def hier_first_tie_high(q, c1, offs, centroids, kid, m):
    return _hier(q, c1, offs, centroids, kid, m, high_j=True)


def hier_returns_position(q, c1, offs, centroids, kid, m):
    return _hier(q, c1, offs, centroids, kid, m, pos_out=True)


def hier_tie_by_position(q, c1, offs, centroids, kid, m):
    return _hier(q, c1, offs, centroids, kid, m, tie_pos=True)


def nearest_by_cosine(x, C):
    C = np.asarray(C, np.float64)
    x = np.asarray(x, np.float64)
    cos = (C @ x) / (np.linalg.norm(C, axis=1) * np.linalg.norm(x) + 1e-300)
    return int(np.argmax(cos))


def nearest_ties_high(x, C):
    d2 = np.sum((np.asarray(C, np.float64) - np.asarray(x, np.float64)) ** 2, axis=1)
    return int(len(d2) - 1 - np.argmin(d2[::-1]))


def update_sum_not_mean(X, assign, C):
    C = np.array(C, np.float64)
    for k in range(C.shape[0]):
        members = np.asarray(X, np.float64)[assign == k]
        if members.shape[0]:
            C[k] = members.sum(axis=0)
    return C


def update_empty_to_zero(X, assign, C):
    C2 = _orig_update(X, assign, C)
    for k in range(C2.shape[0]):
        if not np.any(assign == k):
            C2[k] = 0.0
    return C2


def aggregate_plain_average(assign, a, lse, K):
    a = np.asarray(a, np.float64)
    abar = np.zeros((K, a.shape[1]))
    lz = np.full(K, -np.inf)
    for k in range(K):
        idx = np.nonzero(np.asarray(assign) == k)[0]
        if idx.size:
            abar[k] = a[idx].mean(axis=0)
            lz[k] = np.logaddexp.reduce(np.asarray(lse)[idx])
    return abar, lz


def bounds_drop_last(L, chunks):
    b = _orig_bounds(L, chunks)
    return b[:-1] if len(b) > 1 else b


def compact_reversed(cache, b, g, keep):
    n = keep.shape[0]
    idx = np.nonzero(keep)[0][::-1]
    kept = idx.shape[0]
    for arr in (cache.k, cache.v, cache.pos) + (() if cache.log_beta is None
                                                  else (cache.log_beta,)):
        arr[b, g, :kept] = arr[b, g, :n][idx].copy()
    cache.length[b, g] = kept
    return kept


def phi_identity(x):
    return np.asarray(x, np.float64)


def absorb_no_decay(Mst, bst, K_ev, V_ev, lam):
    return _orig_absorb(Mst, bst, K_ev, V_ev, 1.0)


def absorb_reversed(Mst, bst, K_ev, V_ev, lam):
    return _orig_absorb(Mst, bst, np.asarray(K_ev)[::-1], np.asarray(V_ev)[::-1], lam)


def absorb_kv_swapped(Mst, bst, K_ev, V_ev, lam):
    Mst = np.array(Mst, np.float64)
    bst = np.array(bst, np.float64)
    for k, v in zip(np.asarray(K_ev, np.float64), np.asarray(V_ev, np.float64)):
        Mst = lam * Mst + np.outer(v, OL.phi(k))
        bst = lam * bst + OL.phi(k)
    return Mst, bst


def read_no_stabiliser(Mst, bst, q, W_o, w_g, c_g, eps):
    res, g = _orig_read(Mst, bst, q, W_o, w_g, c_g, eps)
    f = OL.phi(q)
    return res * (float(np.asarray(bst) @ f) + eps), g


def read_gate_flipped(Mst, bst, q, W_o, w_g, c_g, eps):
    res, g = _orig_read(Mst, bst, q, W_o, w_g, c_g, eps)
    return res / g * (1.0 - g), 1.0 - g


def read_no_projection(Mst, bst, q, W_o, w_g, c_g, eps):
    return _orig_read(Mst, bst, q, np.eye(np.asarray(W_o).shape[0]), w_g, c_g, eps)


def _decode_attention(k, v, log_beta, pos, length, q, t, scale=None, head_map=None,
                      default=None):
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None or scale <= 0:
        scale = default(D) if default else 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = head_map(h, G, Hkv) if head_map else h // G
            n = int(length[b][g])
            lb = None if log_beta is None else log_beta[b][g][:n]
            out[b, h], lse[b, h] = OT.attention(q[b, h], k[b][g][:n], v[b][g][:n], lb,
                                                pos[b][g][:n], int(t[b]), scale)
    return out, lse


def decode_attention_h_mod(*a, **kw):
    return _decode_attention(*a, head_map=lambda h, G, Hkv: h % Hkv, **kw)


def decode_attention_sqrt_default(*a, **kw):
    return _decode_attention(*a, default=lambda D: np.sqrt(D), **kw)


def _asm_batched(q, centroids, abar, log_zbar, self_out, self_lse, lookup, head_map=None,
                 first_head=False):
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = centroids.shape[0] if hasattr(centroids, "shape") else len(centroids)
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    idx = np.zeros((B, Hq), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            g = head_map(h, G, Hkv) if head_map else h // G
            c = lookup(q[b, g * G] if first_head else q[b, h], g)
            idx[b, h] = c
            out[b, h], lse[b, h] = OA.asm_merge(self_out[b, h], self_lse[b, h],
                                                abar[g][c], log_zbar[g][c])
    return out, lse, idx


def asm_batched_h_mod(q, C, abar, lz, so, sl):
    return _asm_batched(q, C, abar, lz, so, sl, lambda x, g: _orig_lookup(x, C[g]),
                        head_map=lambda h, G, Hkv: h % Hkv)


def asm_batched_first_head(q, C, abar, lz, so, sl):
    return _asm_batched(q, C, abar, lz, so, sl, lambda x, g: _orig_lookup(x, C[g]),
                        first_head=True)


def asm_hier_batched_h_mod(q, c1, offs, C, kid, m, abar, lz, so, sl):
    return _asm_batched(q, c1, abar, lz, so, sl,
                        lambda x, g: _orig_hier_b(x, c1[g], offs[g], C[g], kid[g], m),
                        head_map=lambda h, G, Hkv: h % Hkv)


def asm_hier_batched_first_head(q, c1, offs, C, kid, m, abar, lz, so, sl):
    return _asm_batched(q, c1, abar, lz, so, sl,
                        lambda x, g: _orig_hier_b(x, c1[g], offs[g], C[g], kid[g], m),
                        first_head=True)


def decode_evict_before_attend(*a, **kw):
    # append, evict, then attend
    cache, qs, k_news, v_news, lb_news, t0, M = a[:7]
    c = cache.copy()
    B = c.length.shape[0]
    steps = []
    for s in range(len(qs)):
        t = np.full(B, t0 + s, dtype=np.int64)
        OE.append_tokens(c, k_news[s], v_news[s], None if lb_news is None else lb_news[s], t)
        c, ev, n_ev = OE.evict_to_budget(c, t, M)
        out, lse = OT.decode_attention(c.values("k"), c.values("v"), c.log_beta, c.pos,
                                       c.length, qs[s], t, kw.get("scale"))
        steps.append((out, lse, ev, n_ev))
    return c, steps


def decode_attend_before_append(*a, **kw):
    # the decode token is left out of its own step's attention
    cache, qs, k_news, v_news, lb_news, t0, M = a[:7]
    c = cache.copy()
    B = c.length.shape[0]
    steps = []
    for s in range(len(qs)):
        t = np.full(B, t0 + s, dtype=np.int64)
        out, lse = OT.decode_attention(c.values("k"), c.values("v"), c.log_beta, c.pos,
                                       c.length, qs[s], t, kw.get("scale"))
        OE.append_tokens(c, k_news[s], v_news[s], None if lb_news is None else lb_news[s], t)
        c, ev, n_ev = OE.evict_to_budget(c, t, M)
        steps.append((out, lse, ev, n_ev))
    return c, steps


def _erase_pages_slip(cache, pages, ranges, keep_empty=False, in_place=False):
    out, pg = cache.copy(), pages.copy()
    B, H = cache.length.shape
    n_er = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for g in range(H):
            table, fill, before, after = [], [], 0, 0
            for i in range(int(pages.n_pages[b, g])):
                p, f = int(pages.table[b, g, i]), int(pages.fill[b, g, i])
                rows = np.arange(32 * p, 32 * p + f)
                keep = OE.erase_plan(cache.pos[b, g, rows], f, ranges[b])
                kept = int(keep.sum())
                before, after = before + f, after + kept
                if kept == 0 and not keep_empty:
                    continue
                if not in_place:
                    for name in ("k", "v", "pos", "log_beta"):
                        a = getattr(out, name)
                        if a is not None:
                            a[b, g, 32 * p:32 * p + kept] = a[b, g, rows[keep]].copy()
                table.append(p)
                fill.append(kept)
            pg.table[b, g, :len(table)] = table
            pg.fill[b, g, :len(fill)] = fill
            pg.n_pages[b, g] = len(table)
            out.length[b, g] = after
            n_er[b, g] = before - after
    return out, pg, n_er


def erase_pages_keeps_empty(cache, pages, ranges):
    return _erase_pages_slip(cache, pages, ranges, keep_empty=True)


def erase_pages_no_compaction(cache, pages, ranges):
    return _erase_pages_slip(cache, pages, ranges, in_place=True)


_orig_paged_append = OE.paged_append


def paged_append_prefers_spare(cache, pages, k_new, v_new, log_beta_new, t, spare):
    full = pages.fill.copy()
    for b in range(full.shape[0]):
        for g in range(full.shape[1]):
            n = int(pages.n_pages[b, g])
            if spare is not None and spare[b, g] >= 0 and n > 0:
                pages.fill[b, g, n - 1] = 32
    st = _orig_paged_append(cache, pages, k_new, v_new, log_beta_new, t, spare)
    for b in range(full.shape[0]):
        for g in range(full.shape[1]):
            n = int(pages.n_pages[b, g])
            for i in range(n - 1):
                pages.fill[b, g, i] = full[b, g, i]
    return st


def paged_slots_full_pages(pages, b, g):
    out = []
    for i in range(int(pages.n_pages[b, g])):
        p = int(pages.table[b, g, i])
        out.extend(range(32 * p, 32 * p + 32))
    return np.asarray(out, dtype=np.int64)


MUTANTS = [
    (OT, "retention_bias", bias_sign_flipped),
    (OT, "retention_bias", bias_dropped),
    (OT, "retention_bias", bias_uses_slot),
    (OT, "retention_bias", bias_ignores_zero_distance),
    (OT, "attention_state", state_bias_scaled),
    (OT, "attention_state", state_no_scale),
    (OT, "attention_state", state_k_for_v),
    (OT, "merge_states", merge_weights_swapped),
    (OT, "merge_states", merge_no_rescale),
    (OE, "retention_keys", keys_negated),
    (OE, "retention_keys", keys_no_distance),
    (OE, "evict_plan", plan_ties_high_first),
    (OE, "evict_plan", plan_off_by_one),
    (OE, "erase_plan", erase_closed),
    (OA, "cosine_lookup", lookup_raw_dot),
    (OA, "cosine_lookup", lookup_last_tie),
    (OA, "asm_merge", asm_merge_linear),
    (OE, "compact_unit", compact_reversed),
    (OA, "hier_lookup", hier_first_level_dot),
    (OA, "hier_lookup", hier_keeps_one_fewer),
    (OA, "hier_lookup", hier_first_tie_high),
    (OA, "hier_lookup", hier_returns_position),
    (OA, "hier_lookup", hier_tie_by_position),
    (OAB, "nearest_centroid", nearest_by_cosine),
    (OAB, "nearest_centroid", nearest_ties_high),
    (OAB, "centroid_update", update_sum_not_mean),
    (OAB, "centroid_update", update_empty_to_zero),
    (OAB, "aggregate_states", aggregate_plain_average),
    (OAB, "chunk_bounds", bounds_drop_last),
    (OL, "phi", phi_identity),
    (OL, "latent_absorb", absorb_no_decay),
    (OL, "latent_absorb", absorb_reversed),
    (OL, "latent_absorb", absorb_kv_swapped),
    (OL, "latent_read", read_no_stabiliser),
    (OL, "latent_read", read_gate_flipped),
    (OL, "latent_read", read_no_projection),
    (OT, "decode_attention", decode_attention_h_mod),
    (OT, "decode_attention", decode_attention_sqrt_default),
    (OA, "asm_lookup_merge", asm_batched_h_mod),
    (OA, "asm_lookup_merge", asm_batched_first_head),
    (OA, "asm_lookup_merge_hier", asm_hier_batched_h_mod),
    (OA, "asm_lookup_merge_hier", asm_hier_batched_first_head),
    (OD, "run_decode_steps", decode_evict_before_attend),
    (OD, "run_decode_steps", decode_attend_before_append),
    (OE, "erase_pages", erase_pages_keeps_empty),
    (OE, "erase_pages", erase_pages_no_compaction),
    (OE, "paged_append", paged_append_prefers_spare),
    (OE, "paged_slots", paged_slots_full_pages),
]


@pytest.mark.parametrize("mod,name,mutant", MUTANTS, ids=lambda x: getattr(x, "__name__", ""))
def test_mutant_fails_a_pin(monkeypatch, mod, name, mutant):
    monkeypatch.setattr(mod, name, mutant)
    failed = []
    for check in pins.ALL:
        try:
            check()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {mutant.__name__}"
