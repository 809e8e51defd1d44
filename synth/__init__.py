"""Seeded synthetic inputs for bounded decode attention.

This module is shared by the float64 oracle's tests and by the HIP path's tests
and benchmark.  It only *draws* inputs: it holds none of the method's arithmetic
(no attention, no retention keys, no eviction, no merge, no lookup).

Distributions follow the five workloads:

* K, V, q ~ N(0, 1); bf16 values are rounded to nearest-even from float64.
* retention: beta = sigmoid(x), x ~ N(2, 1.5) (1.5 is the standard deviation),
  stored as log beta in float32, because the kernels take log beta.
* token positions: 0..n-1 for a fresh cache; the decode token sits at t = n.
* ASM codebooks: centroids ~ N(0,1)^D normalised to unit L2 length in float64,
  then rounded to bf16; stored states abar ~ N(0,1)^D in bf16; log Zbar ~ U(0, 12).
* MEMENTO layout: thinking blocks of uniform integer length in [2048, 16384], each
  followed by a 200-token memento, filling the cache; the last block is the one
  still being written and has no memento.

Host generation uses numpy's PCG64.  Large workloads are drawn on the device
with torch's seeded generator (``device_*`` helpers); their parity checks read
the drawn bits back before any kernel runs.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_bits", "bf16_to_f64", "f32_bits",
    "host_cache", "host_queries", "host_new_tokens", "host_codebook",
    "memento_layout", "memento_pages", "host_paged", "device_cache", "device_queries",
    "device_codebook",
]


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    ctx: int              # tokens in the cache before the decode token
    budget: int           # M, live slots per KV head after eviction
    layers: int
    seed: int
    steps: int = 1        # decode steps (the tiny workload runs 16)
    retention: bool = True   # False: beta == 1 (no log beta array)
    codebook: int = 0     # ASM centroids per KV head (0: no ASM)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def units(self) -> int:
        return self.batch * self.hkv

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "tiny": Workload("tiny", batch=1, hq=8, hkv=2, head_dim=64, dtype="f32",
                     ctx=512, budget=256, layers=1, seed=1001, steps=16),
    "qwen3_8b_32k": Workload("qwen3_8b_32k", batch=16, hq=32, hkv=8, head_dim=128,
                             dtype="bf16", ctx=32768, budget=4096, layers=36,
                             seed=1002),
    "qwen3_32b_128k": Workload("qwen3_32b_128k", batch=8, hq=64, hkv=8, head_dim=128,
                               dtype="bf16", ctx=131072, budget=8192, layers=64,
                               seed=1003),
    "asm_lookup": Workload("asm_lookup", batch=32, hq=32, hkv=8, head_dim=128,
                           dtype="bf16", ctx=2048, budget=1 << 30, layers=36,
                           seed=1004, retention=False, codebook=4096),
    "memento_1m": Workload("memento_1m", batch=1, hq=64, hkv=8, head_dim=128,
                           dtype="bf16", ctx=1 << 20, budget=65536, layers=1,
                           seed=1005, retention=False),
    # two-level ASM lookup: 16K entries per KV head in 128 first-level clusters,
    # the top 16 first-level centroids expanded
    "asm_build": Workload("asm_build", batch=1, hq=32, hkv=8, head_dim=128,
                          dtype="bf16", ctx=16384, budget=1 << 30, layers=1, seed=1007,
                          retention=False, codebook=4096),
    "asm_hier": Workload("asm_hier", batch=32, hq=32, hkv=8, head_dim=128,
                         dtype="bf16", ctx=2048, budget=1 << 30, layers=36,
                         seed=1006, retention=False, codebook=16384),
}
HIER_K1 = 128
HIER_M = 16
# ASM memory construction: per KV head a 16K-token prefix encoded in 4 chunks,
# 16K calibration queries clustered into K = 4096 entries by 10 Lloyd iterations
BUILD_N = 16384
BUILD_CHUNKS = 4
BUILD_ITERS = 10


# --------------------------------------------------------------------------
# dtype helpers (bit-exact, shared by both sides)
# --------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Works on the float64 value directly (no float32 detour, so no double rounding).
    Only finite values within bf16's normal range are expected.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)                   # 8 significant bits, half-to-even
    v = np.ldexp(r, e - 8)                   # exact in float64 and in float32
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def _log_sigmoid_f32(x: np.ndarray) -> np.ndarray:
    # log(1/(1+e^-x)) evaluated stably in float64, stored as float32
    x = np.asarray(x, dtype=np.float64)
    out = np.where(x >= 0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))
    return out.astype(np.float32)


def _draw_values(rng, shape, dtype):
    z = rng.standard_normal(size=shape)
    if dtype == "bf16":
        return bf16_bits(z)
    return z.astype(np.float32)


# --------------------------------------------------------------------------
# host generators (numpy PCG64)
# --------------------------------------------------------------------------
def host_cache(w: Workload, n: int | None = None, cap: int | None = None,
               seed: int | None = None, units: tuple[int, int] | None = None):
    """A fresh cache with n live tokens per KV head at positions 0..n-1.

    Returns a dict of numpy arrays (uint16 bf16 bits or float32 values):
    k, v [B][Hkv][cap][D]; log_beta [B][Hkv][cap] float32 (or None);
    pos [B][Hkv][cap] int32; len [B][Hkv] int32.
    Slots at and beyond n hold zeros.
    """
    n = w.ctx if n is None else n
    cap = n + w.steps if cap is None else cap
    B, H = (w.batch, w.hkv) if units is None else units
    D = w.head_dim
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    vd = np.uint16 if w.dtype == "bf16" else np.float32
    k = np.zeros((B, H, cap, D), vd)
    v = np.zeros((B, H, cap, D), vd)
    k[:, :, :n] = _draw_values(rng, (B, H, n, D), w.dtype)
    v[:, :, :n] = _draw_values(rng, (B, H, n, D), w.dtype)
    log_beta = None
    if w.retention:
        log_beta = np.zeros((B, H, cap), np.float32)
        log_beta[:, :, :n] = _log_sigmoid_f32(rng.normal(2.0, 1.5, size=(B, H, n)))
    pos = np.zeros((B, H, cap), np.int32)
    pos[:, :, :n] = np.arange(n, dtype=np.int32)
    length = np.full((B, H), n, np.int32)
    return {"k": k, "v": v, "log_beta": log_beta, "pos": pos, "len": length}


def host_queries(w: Workload, steps: int | None = None, seed_offset: int = 7,
                 batch: int | None = None):
    """q [steps][B][Hq][D] (bf16 bits or float32)."""
    steps = w.steps if steps is None else steps
    B = w.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    return _draw_values(rng, (steps, B, w.hq, w.head_dim), w.dtype)


def host_new_tokens(w: Workload, steps: int | None = None, seed_offset: int = 13,
                    batch: int | None = None):
    """Per decode step: k_new, v_new [steps][B][Hkv][D], log_beta_new [steps][B][Hkv]."""
    steps = w.steps if steps is None else steps
    B = w.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    k = _draw_values(rng, (steps, B, w.hkv, w.head_dim), w.dtype)
    v = _draw_values(rng, (steps, B, w.hkv, w.head_dim), w.dtype)
    lb = None
    if w.retention:
        lb = _log_sigmoid_f32(rng.normal(2.0, 1.5, size=(steps, B, w.hkv)))
    return k, v, lb


def host_codebook(w: Workload, K: int | None = None, seed_offset: int = 29):
    """ASM codebook per KV head: centroids, abar [Hkv][K][D] bf16 bits; log_zbar [Hkv][K] f32."""
    K = w.codebook if K is None else K
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    c = rng.standard_normal(size=(w.hkv, K, w.head_dim))
    c = c / np.sqrt((c * c).sum(axis=-1, keepdims=True))
    centroids = bf16_bits(c)
    abar = bf16_bits(rng.standard_normal(size=(w.hkv, K, w.head_dim)))
    log_zbar = rng.uniform(0.0, 12.0, size=(w.hkv, K)).astype(np.float32)
    return centroids, abar, log_zbar


def host_hier_codebook(w: Workload, K: int, K1: int, spread: float = 1.0,
                       seed_offset: int = 31):
    """A two-level codebook per KV head, built from latent cluster directions.

    Each of the K entries belongs to one of K1 clusters (drawn uniformly, so some
    clusters may be small or empty); entry = normalise(u_j + spread * N(0, I/D))
    for its cluster's unit direction u_j.  The first-level centroids are the u_j
    themselves.  Entries are stored cluster by cluster (random order inside a
    cluster).  Returns (c1 [Hkv][K1][D], offs [Hkv][K1+1] int32, stored
    [Hkv][K][D], kid [Hkv][K] int32 = original index of each stored entry,
    abar [Hkv][K][D] and log_zbar [Hkv][K] in original order); vectors are bf16
    bits.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset + 7919 * K1))
    H, D = w.hkv, w.head_dim
    u = rng.standard_normal((H, K1, D))
    u /= np.sqrt((u * u).sum(-1, keepdims=True))
    assign = rng.integers(0, K1, size=(H, K))
    x = u[np.arange(H)[:, None], assign] + spread * rng.standard_normal((H, K, D)) / np.sqrt(D)
    x /= np.sqrt((x * x).sum(-1, keepdims=True))
    cent = bf16_bits(x)
    stored = np.empty_like(cent)
    kid = np.empty((H, K), np.int32)
    offs = np.empty((H, K1 + 1), np.int32)
    for g in range(H):
        perm = np.lexsort((rng.permutation(K), assign[g]))
        stored[g] = cent[g, perm]
        kid[g] = perm
        offs[g] = np.searchsorted(assign[g, perm], np.arange(K1 + 1))
    abar = bf16_bits(rng.standard_normal((H, K, D)))
    log_zbar = rng.uniform(0.0, 12.0, size=(H, K)).astype(np.float32)
    return bf16_bits(u), offs, stored, kid, abar, log_zbar, cent


def host_near_queries(w: Workload, entries, noise: float = 0.5, seed_offset: int = 37):
    """Decode queries near stored entries: q = |N(0,1)| scale x (c_k + noise * N(0, I/D))
    for a random entry k of the query head's KV head.  entries: [Hkv][K][D] bf16
    bits (original order).  Returns q [B][Hq][D] bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    H, K, D = entries.shape
    G = w.hq // H
    B = w.batch
    c = bf16_to_f64(entries)
    k = rng.integers(0, K, size=(B, w.hq))
    g = (np.arange(w.hq) // G)[None, :].repeat(B, 0)
    q = c[g, k] + noise * rng.standard_normal((B, w.hq, D)) / np.sqrt(D)
    q *= np.abs(rng.standard_normal((B, w.hq, 1))) + 0.5
    return bf16_bits(q)


def host_asm_build(w: Workload, N: int, L: int | None = None, topics: int = 512,
                   seed_offset: int = 41):
    """Calibration data for building a memory, per KV head.

    Prefix K, V [Hkv][L][D] ~ N(0, 1); calibration queries Q [Hkv][N][D] drawn
    around `topics` random directions: q = 2 (u_topic + 0.6 N(0, I/D)) scaled by
    (|N(0,1)| + 0.5), so that K-means has structure to find.  bf16 bits.
    """
    L = w.ctx if L is None else L
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    H, D = w.hkv, w.head_dim
    Kp = bf16_bits(rng.standard_normal((H, L, D)))
    Vp = bf16_bits(rng.standard_normal((H, L, D)))
    u = rng.standard_normal((H, topics, D))
    u /= np.sqrt((u * u).sum(-1, keepdims=True))
    tpc = rng.integers(0, topics, size=(H, N))
    q = u[np.arange(H)[:, None], tpc] + 0.6 * rng.standard_normal((H, N, D)) / np.sqrt(D)
    q *= 2.0 * (np.abs(rng.standard_normal((H, N, 1))) + 0.5)
    return bf16_bits(q), Kp, Vp


def host_kmeans_init(w: Workload, q: np.ndarray, K: int, seed_offset: int = 43) -> np.ndarray:
    """Initial centroids [H][K][D] float32: K distinct calibration queries of each
    KV head, picked by a seeded permutation (K <= N)."""
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    H, N, _ = q.shape
    vals = bf16_to_f64(q)
    return np.stack([vals[h][rng.permutation(N)[:K]] for h in range(H)]).astype(np.float32)


def host_latent_params(D: int, Hq: int, seed: int, lam: float = 0.9999, eps: float = 1e-6):
    """Synthetic constants of the latent memory read: projection W_o [D][D]
    ~ N(0, 1/D), gate weights w_g [Hq][D] ~ N(0, 1/D), gate bias c_g [Hq] ~ N(0, 1),
    decay lam and eps as given (float32 values)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return {"lam": float(np.float32(lam)), "eps": float(np.float32(eps)),
            "W_o": (rng.standard_normal((D, D)) / np.sqrt(D)).astype(np.float32),
            "w_g": (rng.standard_normal((Hq, D)) / np.sqrt(D)).astype(np.float32),
            "c_g": rng.standard_normal(Hq).astype(np.float32)}


def memento_layout(total: int = 1 << 20, seed: int = 1005, memento: int = 200,
                   lo: int = 2048, hi: int = 16384):
    """Block/memento layout of a reasoning trace filling ``total`` slots.

    Returns (blocks, ranges): blocks is a list of (start, block_len, memento_len);
    ranges is an int32 array [R][2] of half-open position ranges covering every
    completed thinking block (those followed by a memento).  The last block is
    the current one; it has no memento and is not erased.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    blocks = []
    p = 0
    while p < total:
        L = int(rng.integers(lo, hi + 1))
        if p + L + memento >= total:          # current block: runs to the end
            blocks.append((p, total - p, 0))
            break
        blocks.append((p, L, memento))
        p += L + memento
    ranges = np.array([(s, s + L) for (s, L, mlen) in blocks if mlen > 0], np.int32)
    return blocks, ranges.reshape(-1, 2)


def memento_pages(blocks, H: int, seed: int = 1005, page: int = 32, spare: int = 64):
    """Paged layout of a MEMENTO trace in which every thinking block and every
    memento starts on a fresh page (its last page is partly filled).

    Physical pages are drawn per head as a seeded permutation of ``n + spare``
    pages (n: the pages the trace uses), so the table is out of physical order.
    Returns (table [H][n] int32, fill [n] int32, first position of each page [n]
    int32, physical pages per head).
    """
    fill, pos0 = [], []
    for (s, L, mlen) in blocks:
        for (a, m) in ((s, L), (s + L, mlen)):
            for o in range(0, m, page):
                fill.append(min(page, m - o))
                pos0.append(a + o)
    n = len(fill)
    phys = n + spare
    rng = np.random.Generator(np.random.PCG64(seed + 77))
    table = np.stack([rng.permutation(phys)[:n] for _ in range(H)]).astype(np.int32)
    return table, np.array(fill, np.int32), np.array(pos0, np.int32), phys


def host_paged(rng, B: int, H: int, D: int, n_pages_max: int, max_pages: int,
               phys: int, retention: bool = True, full_fill: float = 0.5, gap: int = 2):
    """A small random paged cache: per head a run of pages (count uniform in
    [0, n_pages_max]) on distinct physical pages out of ``phys``, fills uniform in
    1..32 (32 with probability ``full_fill``), positions ascending along the table
    with gaps uniform in [1, gap].  K, V ~ N(0, 1) as bf16 bits over every slot.
    Returns dict k, v (uint16), log_beta, pos, len, table, fill, n_pages."""
    cap = 32 * phys
    k = bf16_bits(rng.standard_normal((B, H, cap, D)))
    v = bf16_bits(rng.standard_normal((B, H, cap, D)))
    lb = (_log_sigmoid_f32((rng.standard_normal((B, H, cap)) * 1.5 + 2.0).astype(np.float32))
          if retention else None)
    pos = np.zeros((B, H, cap), np.int32)
    table = np.full((B, H, max_pages), -1, np.int32)
    fill = np.zeros((B, H, max_pages), np.int32)
    n_pages = np.zeros((B, H), np.int32)
    length = np.zeros((B, H), np.int32)
    for b in range(B):
        for g in range(H):
            n = int(rng.integers(0, n_pages_max + 1))
            perm = rng.permutation(phys)[:n]
            p = int(rng.integers(0, 50))
            for i in range(n):
                f = 32 if rng.random() < full_fill else int(rng.integers(1, 33))
                steps = rng.integers(1, gap + 1, size=f)
                pp = p + np.cumsum(steps)
                pos[b, g, 32 * perm[i]:32 * perm[i] + f] = pp
                p = int(pp[-1])
                table[b, g, i], fill[b, g, i] = perm[i], f
                length[b, g] += f
            n_pages[b, g] = n
    return {"k": k, "v": v, "log_beta": lb, "pos": pos, "len": length, "table": table,
            "fill": fill, "n_pages": n_pages}


# --------------------------------------------------------------------------
# device generators (torch, seeded); used for workloads too large for the host
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def device_cache(w: Workload, layer: int, n: int | None = None, cap: int | None = None,
                 device: str = "cuda", out: dict | None = None):
    """Draw one layer's cache on the device.  Deterministic in (seed, layer).

    The default capacity is n + steps rounded up to a multiple of 32 slots.

    Returns a dict of torch tensors: k, v [B][Hkv][cap][D] (bfloat16 or float32),
    log_beta [B][Hkv][cap] float32 or None, pos int32, len int32.
    If ``out`` is given its tensors are filled in place.
    """
    torch = _torch()
    n = w.ctx if n is None else n
    cap = ceil_div(n + w.steps, 32) * 32 if cap is None else cap
    B, H, D = w.batch, w.hkv, w.head_dim
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000003 + layer)
    if out is None:
        out = {
            "k": torch.empty((B, H, cap, D), dtype=tdt, device=device),
            "v": torch.empty((B, H, cap, D), dtype=tdt, device=device),
            "log_beta": (torch.empty((B, H, cap), dtype=torch.float32, device=device)
                         if w.retention else None),
            "pos": torch.empty((B, H, cap), dtype=torch.int32, device=device),
            "len": torch.empty((B, H), dtype=torch.int32, device=device),
        }
    # bf16 values: draw float32 normals and round to nearest-even bf16
    for name in ("k", "v"):
        t = out[name]
        for b in range(B):      # per batch row bounds the float32 staging buffer
            z = torch.randn((H, n, D), generator=g, device=device, dtype=torch.float32)
            t[b, :, :n].copy_(z.to(tdt))
            del z
        if cap > n:
            t[:, :, n:].zero_()
    if w.retention:
        x = torch.randn((B, H, n), generator=g, device=device, dtype=torch.float32)
        x = x * 1.5 + 2.0
        out["log_beta"][:, :, :n] = torch.nn.functional.logsigmoid(x)
        if cap > n:
            out["log_beta"][:, :, n:].zero_()
    out["pos"][:, :, :n] = torch.arange(n, dtype=torch.int32, device=device)
    if cap > n:
        out["pos"][:, :, n:].zero_()
    out["len"].fill_(n)
    return out


def device_queries(w: Workload, layer: int, device: str = "cuda", step: int = 0):
    torch = _torch()
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 7919 + layer * 131 + step)
    q = torch.randn((w.batch, w.hq, w.head_dim), generator=g, device=device)
    k = torch.randn((w.batch, w.hkv, w.head_dim), generator=g, device=device)
    v = torch.randn((w.batch, w.hkv, w.head_dim), generator=g, device=device)
    lb = None
    if w.retention:
        x = torch.randn((w.batch, w.hkv), generator=g, device=device) * 1.5 + 2.0
        lb = torch.nn.functional.logsigmoid(x)
    return q.to(tdt), k.to(tdt), v.to(tdt), lb


def device_codebook(w: Workload, layer: int, device: str = "cuda"):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 104729 + layer)
    c = torch.randn((w.hkv, w.codebook, w.head_dim), generator=g, device=device,
                    dtype=torch.float64)
    c = c / c.square().sum(-1, keepdim=True).sqrt()
    abar = torch.randn((w.hkv, w.codebook, w.head_dim), generator=g, device=device)
    lz = torch.rand((w.hkv, w.codebook), generator=g, device=device) * 12.0
    return c.to(torch.bfloat16), abar.to(torch.bfloat16), lz.float()


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)
