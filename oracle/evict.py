"""Float64 retention-score eviction, MEMENTO range erasure and stable compaction.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

Cache rows are moved as raw storage values (float32, or bf16 bit patterns held
as uint16), so a compacted layout can be compared bit for bit.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def _bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32) \
        .astype(np.float64)


@dataclasses.dataclass
class Cache:
    """One layer's KV cache.

    k, v      [B][Hkv][cap][D] float32 values, or bf16 bit patterns as uint16
    log_beta  [B][Hkv][cap] float32, or None (beta == 1)
    pos       [B][Hkv][cap] int32 absolute token positions of the slots
    length    [B][Hkv] int32 live slots; slots at and beyond it are unspecified
    """
    k: np.ndarray
    v: np.ndarray
    log_beta: np.ndarray | None
    pos: np.ndarray
    length: np.ndarray

    @classmethod
    def from_arrays(cls, d):
        lb = d.get("log_beta")
        return cls(np.array(d["k"]), np.array(d["v"]),
                   None if lb is None else np.array(lb, dtype=np.float32),
                   np.array(d["pos"], dtype=np.int32), np.array(d["len"], dtype=np.int32))

    def copy(self):
        return Cache(self.k.copy(), self.v.copy(),
                     None if self.log_beta is None else self.log_beta.copy(),
                     self.pos.copy(), self.length.copy())

    def values(self, which):
        """float64 view of k or v (exact upcast of the stored values)."""
        a = getattr(self, which)
        if a.dtype == np.uint16:
            return _bf16_bits_to_f64(a)
        return a.astype(np.float64)


def retention_keys(log_beta, pos, t):
    """Eviction key of every token: the log of its retention score beta_i^(t-i).

    "Cache What Lasts" section 2.2 (inference) evicts the token whose current
    retention score beta_i^(t-i) is lowest.  That power underflows to 0 in any
    float format long before t-i reaches cache lengths, so tokens are ranked by
    the monotone equivalent kappa_i = (t-i) * log beta_i.  With log beta stored
    in float32 (24-bit significand) and |t-i| < 2^29 the float64 product is
    exact.  kappa is +0 at distance 0 and when there is no retention array; -0
    is the same key as +0.
    """
    pos = np.asarray(pos, dtype=np.int64)
    if log_beta is None:
        return np.zeros(pos.shape, dtype=np.float64)
    dist = (np.int64(t) - pos).astype(np.float64)
    lb = np.asarray(log_beta, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        key = dist * lb
    key = np.where(dist == 0.0, 0.0, key)
    return key + 0.0          # -0.0 + 0.0 == +0.0


def evict_plan(log_beta, pos, n, t, M):
    """Which of a head's n live slots survive eviction to budget M.

    If n > M the n - M tokens with the lowest key are evicted in one call (the
    page speaks of one token at a time; a cache over budget by more than one
    needs all of them removed).  Ties in the key go to the lower position
    first, so with beta == 1 the newest M tokens stay (a sliding window).
    Returns (keep bool[n], evicted positions ascending int32).
    """
    keep = np.ones(n, dtype=bool)
    if n <= M:
        return keep, np.zeros(0, dtype=np.int32)
    lb = None if log_beta is None else np.asarray(log_beta)[:n]
    p = np.asarray(pos)[:n].astype(np.int64)
    key = retention_keys(lb, p, t)
    order = np.lexsort((p, key))          # by key, then by position
    gone = order[: n - M]
    keep[gone] = False
    return keep, np.sort(p[gone]).astype(np.int32)


def erase_plan(pos, n, ranges):
    """Slots of one head that survive MEMENTO erasure.

    The MEMENTO page removes a finished thinking block's KV entries once its
    memento is written.  Ranges are half-open position intervals [s, e); a slot
    is kept iff its position lies in none of them.
    """
    p = np.asarray(pos)[:n].astype(np.int64)
    keep = np.ones(n, dtype=bool)
    for s, e in np.asarray(ranges, dtype=np.int64).reshape(-1, 2):
        keep &= ~((p >= s) & (p < e))
    return keep


def compact_unit(cache: Cache, b: int, g: int, keep):
    """Move the kept rows of head (b, g), in slot order, to slots [0, kept).

    Stable (order preserving), so slot order stays position order.  Rows at and
    beyond the new length are left as they were (unspecified).
    """
    n = keep.shape[0]
    idx = np.nonzero(keep)[0]
    kept = idx.shape[0]
    for arr in (cache.k, cache.v, cache.pos) + (() if cache.log_beta is None
                                                  else (cache.log_beta,)):
        rows = arr[b, g, :n][idx].copy()
        arr[b, g, :kept] = rows
    cache.length[b, g] = kept
    return kept


def evict_to_budget(cache: Cache, t, M):
    """Evict every over-budget head to M live slots and compact, on a copy.

    Returns (new cache, evicted positions [B][Hkv] list of arrays, n_evicted).
    """
    out = cache.copy()
    B, H = cache.length.shape
    ev = [[None] * H for _ in range(B)]
    n_ev = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for g in range(H):
            n = int(cache.length[b, g])
            lb = None if cache.log_beta is None else cache.log_beta[b, g]
            keep, gone = evict_plan(lb, cache.pos[b, g], n, int(t[b]), M)
            compact_unit(out, b, g, keep)
            ev[b][g] = gone
            n_ev[b, g] = gone.shape[0]
    return out, ev, n_ev


def erase_ranges(cache: Cache, ranges):
    """Erase position ranges (per sequence, all KV heads) and compact, on a copy.

    ranges[b] is an array [R_b][2] of half-open position ranges of sequence b.
    Erasure is textual, so it applies to every KV head of the sequence.
    Returns (new cache, n_erased [B][Hkv]).
    """
    out = cache.copy()
    B, H = cache.length.shape
    n_er = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for g in range(H):
            n = int(cache.length[b, g])
            keep = erase_plan(cache.pos[b, g], n, ranges[b])
            kept = compact_unit(out, b, g, keep)
            n_er[b, g] = n - kept
    return out, n_er


def append_tokens(cache: Cache, k_new, v_new, log_beta_new, t):
    """Write each head's new token at slot len with position t[b]; len += 1 (in place)."""
    B, H = cache.length.shape
    for b in range(B):
        for g in range(H):
            s = int(cache.length[b, g])
            if s >= cache.k.shape[2]:
                raise ValueError("cache full")
            cache.k[b, g, s] = k_new[b, g]
            cache.v[b, g, s] = v_new[b, g]
            if cache.log_beta is not None:
                cache.log_beta[b, g, s] = log_beta_new[b, g]
            cache.pos[b, g, s] = t[b]
            cache.length[b, g] = s + 1
    return cache


# ---------------------------------------------------------------- paged form
# A paged cache keeps each head's tokens in pages of 32 slots.  The page table lists
# a head's pages in position order; physical page p of a head is slots
# [32p, 32p + 32) of that head's arrays, and a page holds its live tokens in its first
# `fill` slots.  The token sequence of a head is its pages' live rows in table order.
PAGE = 32
_ROW_ARRAYS = ("k", "v", "pos")


@dataclasses.dataclass
class Pages:
    """table, fill [B][Hkv][max_pages] int32; n_pages [B][Hkv] int32."""
    table: np.ndarray
    fill: np.ndarray
    n_pages: np.ndarray

    def copy(self):
        return Pages(self.table.copy(), self.fill.copy(), self.n_pages.copy())


def paged_slots(pages: Pages, b: int, g: int):
    """Slots of head (b, g)'s live tokens, in sequence order."""
    out = []
    for i in range(int(pages.n_pages[b, g])):
        p = int(pages.table[b, g, i])
        out.extend(range(PAGE * p, PAGE * p + int(pages.fill[b, g, i])))
    return np.asarray(out, dtype=np.int64)


def paged_view(cache: Cache, pages: Pages):
    """The contiguous cache holding each head's token sequence at slots [0, len)."""
    out = cache.copy()
    B, H = cache.length.shape
    for b in range(B):
        for g in range(H):
            idx = paged_slots(pages, b, g)
            n = idx.shape[0]
            for name in _ROW_ARRAYS + (() if cache.log_beta is None else ("log_beta",)):
                getattr(out, name)[b, g, :n] = getattr(cache, name)[b, g][idx]
            out.length[b, g] = n
    return out


def erase_pages(cache: Cache, pages: Pages, ranges):
    """MEMENTO erasure on a paged cache, on copies; returns (cache, pages, n_erased).

    The kept tokens are those of erase_plan (position in no range).  Removal is by
    page: a page with no kept row leaves the table, and a page with some keeps them
    in order in its first slots (rows of other pages do not move).  The table keeps
    the remaining pages in order; len is the kept total.
    """
    out, pg = cache.copy(), pages.copy()
    B, H = cache.length.shape
    n_er = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for g in range(H):
            table, fill = [], []
            before = after = 0
            for i in range(int(pages.n_pages[b, g])):
                p, f = int(pages.table[b, g, i]), int(pages.fill[b, g, i])
                rows = np.arange(PAGE * p, PAGE * p + f)
                keep = erase_plan(cache.pos[b, g, rows], f, ranges[b])
                kept = int(keep.sum())
                before += f
                after += kept
                if kept == 0:
                    continue
                for arr in (out.k, out.v, out.pos) + (() if out.log_beta is None
                                                      else (out.log_beta,)):
                    arr[b, g, PAGE * p:PAGE * p + kept] = arr[b, g, rows[keep]].copy()
                table.append(p)
                fill.append(kept)
            pg.table[b, g, :len(table)] = table
            pg.fill[b, g, :len(fill)] = fill
            pg.n_pages[b, g] = len(table)
            out.length[b, g] = after
            n_er[b, g] = before - after
    return out, pg, n_er


def paged_append(cache: Cache, pages: Pages, k_new, v_new, log_beta_new, t, spare):
    """Each head's decode token into its last page when that has a free slot, else
    into its free page spare[b][g] added to the end of the table (in place).
    Returns [B][Hkv] bool: stored (False where the head had no room)."""
    B, H = cache.length.shape
    max_pages = pages.table.shape[2]
    stored = np.zeros((B, H), dtype=bool)
    for b in range(B):
        for g in range(H):
            n = int(pages.n_pages[b, g])
            if n > 0 and pages.fill[b, g, n - 1] < PAGE:
                p, r = int(pages.table[b, g, n - 1]), int(pages.fill[b, g, n - 1])
                pages.fill[b, g, n - 1] = r + 1
            elif spare is not None and spare[b, g] >= 0 and n < max_pages:
                p, r = int(spare[b, g]), 0
                pages.table[b, g, n] = p
                pages.fill[b, g, n] = 1
                pages.n_pages[b, g] = n + 1
            else:
                continue
            s = PAGE * p + r
            cache.k[b, g, s] = k_new[b, g]
            cache.v[b, g, s] = v_new[b, g]
            if cache.log_beta is not None:
                cache.log_beta[b, g, s] = log_beta_new[b, g]
            cache.pos[b, g, s] = t[b]
            cache.length[b, g] += 1
            stored[b, g] = True
    return stored
