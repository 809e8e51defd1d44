"""Helpers for GPU parity tests: host<->device copies of exact bits, tolerance checks."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bounded_decode_attention_amd as kvb
import oracle

DEV = "cuda"
ATOL_REL = 2e-3   # max relative error per (b, h): |out - ref|_inf / |ref|_inf
LSE_TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype=None):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_host(t):
    """device tensor -> numpy with the exact stored bits (bf16 -> uint16)."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def dev_cache(d):
    return kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]), to_dev(d["pos"]),
                       to_dev(d["len"]))


def host_dict(c: kvb.KVCache):
    return {"k": to_host(c.k), "v": to_host(c.v), "log_beta": to_host(c.log_beta),
            "pos": to_host(c.pos), "len": to_host(c.length)}


def values(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def check_attention(out, lse, ref_out, ref_lse, what=""):
    """Per (b, h): inf-norm relative error <= 2e-3 and |lse - ref| <= 2e-3;
    empty heads (ref lse = -inf) must give out = 0 and lse = -inf."""
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    B, H = ref_lse.shape
    worst = 0.0
    for b in range(B):
        for h in range(H):
            if ref_lse[b, h] == -np.inf:
                assert lse[b, h] == -np.inf, f"{what} ({b},{h}) lse {lse[b, h]} for empty head"
                assert np.all(out[b, h] == 0), f"{what} ({b},{h}) non-zero out for empty head"
                continue
            den = np.max(np.abs(ref_out[b, h]))
            err = np.max(np.abs(out[b, h] - ref_out[b, h])) / max(den, 1e-30)
            worst = max(worst, err)
            assert err <= ATOL_REL, f"{what} ({b},{h}) rel err {err:.3e}"
            assert abs(lse[b, h] - ref_lse[b, h]) <= LSE_TOL, \
                f"{what} ({b},{h}) lse {lse[b, h]} vs {ref_lse[b, h]}"
    return worst


def check_layout(got: dict, ref: oracle.Cache, what=""):
    """Bit-exact live layout: len, and k, v, log_beta, pos of every live slot."""
    assert np.array_equal(got["len"], ref.length), f"{what} len {got['len']} vs {ref.length}"
    B, H = ref.length.shape
    for b in range(B):
        for g in range(H):
            n = int(ref.length[b, g])
            for name in ("k", "v", "pos"):
                a = got[name][b, g, :n]
                r = getattr(ref, name)[b, g, :n]
                if not np.array_equal(a.view(np.uint8) if a.dtype != np.int32 else a,
                                      r.view(np.uint8) if r.dtype != np.int32 else r):
                    bad = np.nonzero(np.any((a != r).reshape(n, -1), axis=1))[0]
                    raise AssertionError(f"{what} ({b},{g}) {name} differs at slots {bad[:10]}")
            if ref.log_beta is not None:
                a = got["log_beta"][b, g, :n].view(np.uint32)
                r = ref.log_beta[b, g, :n].view(np.uint32)
                assert np.array_equal(a, r), f"{what} ({b},{g}) log_beta differs"


def oracle_attention(d, q, t, scale=None):
    """Oracle attention over a host cache dict (exact upcasts)."""
    return oracle.decode_attention(values(d["k"]), values(d["v"]), d["log_beta"], d["pos"],
                                   d["len"], values(q), t, scale)


def snapshot_rows(c: kvb.KVCache, keep_idx):
    """Copy the rows at the given slots (per head) to the host, from the device,
    before a compaction overwrites them.  keep_idx[(b, g)] = int array of slots."""
    snap = {}
    for (b, g), idx in keep_idx.items():
        it = torch.from_numpy(np.asarray(idx, np.int64)).cuda()
        snap[(b, g)] = {
            "k": to_host(c.k[b, g].index_select(0, it)),
            "v": to_host(c.v[b, g].index_select(0, it)),
            "pos": to_host(c.pos[b, g].index_select(0, it)),
            "log_beta": None if c.log_beta is None else to_host(c.log_beta[b, g].index_select(0, it)),
        }
    return snap


def check_compacted(c: kvb.KVCache, snap, what=""):
    """Head (b, g) must hold exactly the snapshot rows, in order, in slots [0, kept)."""
    lens = to_host(c.length)
    for (b, g), s in snap.items():
        n = s["pos"].shape[0]
        assert lens[b, g] == n, f"{what} ({b},{g}) len {lens[b, g]} vs {n}"
        for name in ("k", "v", "pos", "log_beta"):
            if s[name] is None:
                continue
            got = to_host(getattr(c, name)[b, g, :n])
            ok = np.array_equal(got.view(np.uint8), s[name].view(np.uint8))
            if not ok:
                bad = np.nonzero(np.any((got != s[name]).reshape(n, -1), axis=1))[0]
                raise AssertionError(f"{what} ({b},{g}) {name} differs at slots {bad[:10]}")
