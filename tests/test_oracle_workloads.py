"""Oracle checks on the workloads' own shapes (CPU only)."""
import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_indexmem_bytes():
    g = json.load(open(os.path.join(GOLDEN, "indexmem_kv_bytes.json")))
    a = g["assumed_architecture"]
    per_tok = oracle.kv_bytes_per_token(a["layers"], a["kv_heads"], a["head_dim"],
                                        a["bytes_per_value"])
    assert per_tok * g["tokens"] == g["kv_bytes_total"]
    assert abs(g["kv_bytes_total"] / 2**30 - 320) < 1e-9


def test_memento_erase_closed_form():
    """Kept = 200 per completed block + the current block, on a reduced layout."""
    for total, seed in ((1 << 17, 3), (1 << 18, 4), (1 << 20, 1005)):
        blocks, ranges = synth.memento_layout(total=total, seed=seed)
        pos = np.arange(total, dtype=np.int32)
        keep = oracle.erase_plan(pos, total, ranges)
        completed = sum(1 for b in blocks if b[2] > 0)
        assert keep.sum() == 200 * completed + blocks[-1][1]
        # every kept position is a memento or the current block
        kp = pos[keep]
        mem = np.zeros(total, bool)
        for s, L, m in blocks:
            mem[s + L: s + L + m] = True
        mem[blocks[-1][0]:] = True
        assert mem[kp].all() and mem.sum() == kp.size


def test_tiny_decode_loop():
    """Tiny workload: 16 steps; 513 -> 256 on the first step, 257 -> 256 after."""
    w = synth.WORKLOADS["tiny"]
    c = oracle.Cache.from_arrays(synth.host_cache(w))
    qs = synth.host_queries(w).astype(np.float64)
    kn, vn, lbn = synth.host_new_tokens(w)
    final, steps = oracle.run_decode_steps(c, qs, kn, vn, lbn, w.ctx, w.budget)
    assert steps[0][3].tolist() == [[257, 257]]
    for s in range(1, w.steps):
        assert steps[s][3].tolist() == [[1, 1]]
    assert final.length.tolist() == [[256, 256]]
    # every step's decode token survives (distance 0 has the largest key)
    for g in range(w.hkv):
        assert final.pos[0, g, 255] == w.ctx + w.steps - 1
        assert np.all(np.diff(final.pos[0, g, :256]) > 0)
    # outputs are convex combinations of V rows: finite, lse finite
    for out, lse, _, _ in steps:
        assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_split_identity_on_workload_shapes():
    """Split into 64-token blocks (any count) merges back to full attention."""
    w = synth.WORKLOADS["tiny"]
    d = synth.host_cache(w)
    k = d["k"][0, 0, :512].astype(np.float64)
    v = d["v"][0, 0, :512].astype(np.float64)
    q = synth.host_queries(w)[0, 0, 0].astype(np.float64)
    lb = d["log_beta"][0, 0, :512]
    pos = d["pos"][0, 0, :512]
    full = oracle.attention(q, k, v, lb, pos, 512, 0.125)
    for S in (1, 32, 64, 100, 512, 600):
        bounds = list(range(0, 512, S)) + [512]
        o, l, _ = oracle.split_attention(q, k, v, lb, pos, 512, 0.125, bounds)
        assert np.max(np.abs(o - full[0])) < 1e-12 and abs(l - full[1]) < 1e-12


def test_hier_workload_matches_linear_on_near_queries():
    """On the two-level workload's queries (each near a stored entry), expanding the
    top 16 of 128 first-level clusters finds the linear lookup's entry (the pages
    report this for top-16 expansion); a sample of 64 queries."""
    w = synth.WORKLOADS["asm_hier"]
    c1, offs, stored, kid, _, _, cent = synth.host_hier_codebook(w, w.codebook, synth.HIER_K1)
    q = synth.bf16_to_f64(synth.host_near_queries(w, cent))
    G = w.hq // w.hkv
    agree = 0
    for n, (b, h) in enumerate([(b, h) for b in range(2) for h in range(w.hq)]):
        g = h // G
        lin = oracle.cosine_lookup(q[b, h], synth.bf16_to_f64(cent[g]))
        hi = oracle.hier_lookup(q[b, h], synth.bf16_to_f64(c1[g]), offs[g],
                                synth.bf16_to_f64(stored[g]), kid[g], synth.HIER_M)
        agree += lin == hi
    assert agree >= 62, agree
