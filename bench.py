#!/usr/bin/env python3
"""Decode-step benchmark: bounded-KV decode attention + eviction at 32K context.

One step = one decode step of a 36-layer Qwen3-8B-like stack (batch 16, 32 query
heads / 8 KV heads, head_dim 128, bf16 K/V/q, fp32 accumulation) over a 32768-
token cache per sequence: per layer, append the decode token (t = 32768), run
retention-biased GQA attention over all 32769 live tokens, evict every KV head
to the budget M = 4096 and compact the cache in place.  Inputs are seeded and
synthetic (K, V, q ~ N(0,1) in bf16; beta = sigmoid(N(2, 1.5))) and resident in
HBM before the timed region.  Eviction is destructive, so the first M slots of
every layer (the only ones compaction writes) are restored from a pristine copy
between steps, outside the timed region.

Prints one JSON line.  --gpus N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bounded-KV decode attn: KV GB/s vs HBM peak; decode steps/s at 32K ctx"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_split_qwen3_8b_32k_traffic.json")
STEADY_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_split_steady_m4096_traffic.json")


ATTN_SRC = os.path.join(ROOT, "bounded_decode_attention_amd", "csrc", "attn_decode.hip")
KERNEL_BEGIN = "// ------------------------------------------------------------------ MFMA split"
KERNEL_END = "// The splits plus the ASM lookup's candidate scan in one launch"


def kernel_digest(path=ATTN_SRC):
    """Digest of the split kernels' device code (the attention source between the
    two markers: the MFMA split kernels, the pipelined kernel and its tile
    helpers), so that host-side edits elsewhere in the file keep recorded counters
    valid and any edit of the kernels themselves voids them."""
    text = open(path).read()
    i, j = text.find(KERNEL_BEGIN), text.find(KERNEL_END)
    if i < 0 or j < i:
        return None
    return hashlib.sha256(text[i:j].encode()).hexdigest()[:16]


def recorded_traffic(path, **match):
    """HBM bytes per launch recorded from FETCH_SIZE / WRITE_SIZE counters, if they
    were taken on the split kernels' code as it is now and in the same
    configuration; else None."""
    if not os.path.exists(path):
        return None
    tr = json.load(open(path))
    if tr.get("kernel_sha") != kernel_digest():
        return None
    if any(tr.get(k) != v for k, v in match.items()):
        return None
    return tr.get("traffic_bytes")


def algorithmic_bytes(w, n, moved_rows):
    """Bytes the step must touch once: K and V rows, log beta and positions of
    every live slot, moved rows (read + write of K, V, log beta, pos), q in,
    out + lse out.  Split-K partial states are overhead and not counted."""
    U, D, e = w.units, w.head_dim, w.elem_bytes
    attn = U * n * 2 * D * e + U * n * 8 + w.batch * w.hq * D * e + w.batch * w.hq * (D + 1) * 4
    moves = moved_rows * 2 * (2 * D * e + 8)
    return attn, moves


def cpu_baseline(w, host_units, t, M, budget_s=12.0, gpu_res=None):
    """The float64 oracle, as it stands, on whole heads (append + attention for the
    head's query group + eviction + compaction), the heads taken in turn (again from
    the first once all were run) until ``budget_s`` of CPU work and every head was
    run once; the time per head is extrapolated to the full step (units x layers).

    With ``gpu_res`` (the timed step's results on the same inputs, per layer), each
    head's first oracle run is also compared with them, outside the timed part: the
    compacted layout (len, and K, V, log beta, pos of every kept slot) bit for bit,
    and every query head's output and lse within 2e-3."""
    import numpy as np

    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    if not host_units:
        return None
    done = 0
    elapsed = 0.0
    checked = set()
    worst = 0.0
    for i, (layer, b, g, k, v, lb, pos, n, q, kn, vn, lbn) in enumerate(
            itertools.cycle(host_units)):
        t0 = time.perf_counter()
        c = oracle.Cache(k[None, None].copy(), v[None, None].copy(), lb[None, None].copy(),
                         pos[None, None].copy(), np.array([[n]], np.int32))
        oracle.append_tokens(c, kn[None, None], vn[None, None], np.array([[lbn]], np.float32),
                             np.array([t]))
        ro, rl = oracle.decode_attention(c.values("k"), c.values("v"), c.log_beta, c.pos,
                                         c.length, ((q.astype(np.uint32) << 16)
                                                    .view(np.float32).astype(np.float64))[None],
                                         np.array([t]))
        ce, _, _ = oracle.evict_to_budget(c, np.array([t]), M)
        elapsed += time.perf_counter() - t0
        done += 1
        u = i % len(host_units)
        if gpu_res is not None and u not in checked:
            r = gpu_res[layer]
            kept = int(ce.length[0, 0])
            assert r["len"][b, g] == kept, f"layer {layer} head ({b},{g}): len"
            for name in ("k", "v", "log_beta", "pos"):
                got = r[name][b, g, :kept]
                want = getattr(ce, name)[0, 0, :kept]
                assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), \
                    f"layer {layer} head ({b},{g}): compacted {name} differs from the oracle"
            G = w.group
            for j in range(G):
                o, l = r["out"][b, g * G + j], r["lse"][b, g * G + j]
                err = float(np.max(np.abs(o - ro[0, j])) / np.max(np.abs(ro[0, j])))
                assert err <= 2e-3 and abs(float(l) - rl[0, j]) <= 2e-3, \
                    f"layer {layer} query head ({b},{g * G + j}): rel err {err:.2e}"
                worst = max(worst, err)
            checked.add(u)
        if elapsed >= budget_s and done >= len(host_units):
            break
    unit_s = elapsed / done
    step_s = unit_s * w.units * w.layers
    layers = sorted({hu[0] for hu in host_units})
    res = {"value": 1.0 / step_s, "unit": "decode steps/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} runs over the {len(host_units)} whole KV heads of layers "
                     f"{layers} ({host_units[0][7] + 1} tokens, {w.group} query heads each: "
                     f"append + attention + eviction to {M} + compaction), {elapsed:.1f} s, "
                     f"extrapolated to {w.units} heads x {w.layers} layers",
           "affinity_cpus": len(os.sched_getaffinity(0))}
    if gpu_res is not None:
        res["checked_against_gpu"] = {
            "what": "the timed step replayed on restored inputs: compacted layouts bit for "
                    "bit, attention out/lse within 2e-3",
            "kv_heads": len(checked), "max_rel_err": float(f"{worst:.3e}")}
    return res


def steady_bench(args):
    """Steady-state decode of the 32K workload's model shape under its budget: every
    KV head of the 36 layers holds M = 4096 tokens; a step appends one token per
    layer, attends over M + 1, evicts the lowest-retention token and compacts.  Each
    head has a first-slot entry (kvb_cache.start; its slots form a ring) unless
    --no-start, so the compaction moves the shorter side of the evicted slot (the
    rows before it up one slot, or the rows after it down one) instead of always the
    rows after it.  Default schedule (fill): one kv_attn_decode_evict_one call per
    layer, whose splits also select each head's eviction and whose merge writes the
    decode token into the evicted slot (one row per head; the slots then hold the
    live tokens out of position order, and the heads need no start array);
    --schedule plan_one keeps position order: kv_attn_decode_plan_one, then
    kv_evict_one_apply's shift on a second stream beside the next layer's attention;
    fused_append: a separate eviction plan and compaction there instead;
    both_beside: separate append, the plan beside the layer's own attention;
    deferred: all compactions after the last attention.  Each head's attention is
    cut into 16 splits with fill, 32 otherwise (--splits to change; finer splits
    share the GPU better with a second stream's compaction).  The whole step is
    captured once in a HIP graph and
    replayed (t advances on the device).  A second, eager run of the same steps with
    the library's HIP-event trace gives the per-kernel split."""
    import dataclasses

    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.layers:
        w = dataclasses.replace(w, layers=args.layers)
    L, M, B = w.layers, w.budget, w.batch
    print(f"# generating {L} layers of {w.name} with {M} tokens per KV head", file=sys.stderr,
          flush=True)
    fill = args.schedule in (None, "fill")  # the default here
    plan1 = args.schedule == "plan_one"
    # fill moves no rows, so its heads need no first-slot array (and without one the
    # attention reads log beta and pos 16 bytes at a time)
    use_start = not args.no_start and not fill
    kvs, qs = [], []
    for layer in range(L):
        d = synth.device_cache(w, layer, n=M, cap=M + 32)
        if use_start:
            d["start"] = torch.zeros((B, w.hkv), dtype=torch.int32, device="cuda")
        kvs.append(kvb.KVCache.from_dict(d))
        qs.append(synth.device_queries(w, layer))
    out = torch.empty((B, w.hq, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, w.hq), dtype=torch.float32, device="cuda")
    P = args.splits or (16 if fill else 32)
    ws_a = torch.empty(kvb.kv_attn_decode_evict_one_workspace(kvs[0], w.hq, P) if fill
                       else kvb.kv_attn_decode_workspace(kvs[0], w.hq, P), dtype=torch.uint8,
                       device="cuda")
    if plan1:
        ws_e = [torch.empty(kvb.kv_evict_one_workspace(kvs[0], P), dtype=torch.uint8,
                            device="cuda") for _ in range(L)]
    else:
        ws_e = [torch.empty(kvb.kv_evict_workspace(kvs[0], M), dtype=torch.uint8,
                            device="cuda") for _ in range(L)]
    nev = torch.empty((L, B, w.hkv), dtype=torch.int32, device="cuda")
    t = torch.full((B,), M, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    appended = [torch.cuda.Event() for _ in range(L)]
    attended = [torch.cuda.Event() for _ in range(L)]
    planned = [torch.cuda.Event() for _ in range(L)]
    deferred = args.schedule == "deferred"
    fused_append = args.schedule == "fused_append"
    one = args.schedule == "evict_one"

    def step(ev=None):
        # ev: optional [L][B][Hkv][1] int32, each layer's evicted position per head
        main = torch.cuda.current_stream()
        for layer in range(L):
            q, kn, vn, lb = qs[layer]
            evl = None if ev is None else ev[layer]
            if fill:
                # one call: attention, decode token, eviction (the decode token takes
                # the evicted slot)
                kvb.kv_attn_decode_evict_one(kvs[layer], q, t, M, k_new=kn, v_new=vn,
                                             log_beta_new=lb, num_splits=P, out=out, lse=lse,
                                             evicted_pos=evl, n_evicted=nev[layer], ws=ws_a,
                                             stream=main)
                continue
            if plan1:
                # the attention call appends the decode token and plans each head's
                # eviction; the layer's order-keeping shift follows it on the side
                # stream, beside the next attention
                kvb.kv_attn_decode_plan_one(kvs[layer], q, t, ws_e[layer], k_new=kn, v_new=vn,
                                            log_beta_new=lb, num_splits=P, out=out, lse=lse,
                                            ws=ws_a, stream=main)
                attended[layer].record(main)
                side.wait_event(attended[layer])
                kvb.kv_evict_one_apply(kvs[layer], t, M, ws_e[layer], evicted_pos=evl,
                                       n_evicted=nev[layer], stream=side)
                continue
            if one:
                # the attention call appends the decode token; the layer's eviction
                # (one launch) follows it on the side stream, beside the next attention
                kvb.kv_attn_decode(kvs[layer], q, t, k_new=kn, v_new=vn, log_beta_new=lb,
                                   num_splits=P, out=out, lse=lse, ws=ws_a, stream=main)
                attended[layer].record(main)
                side.wait_event(attended[layer])
                kvb.kv_evict_one(kvs[layer], t, M, evicted_pos=evl, n_evicted=nev[layer],
                                 stream=side)
                continue
            if fused_append:
                # the attention call appends the decode token; the layer's plan and
                # compaction follow it on the side stream, beside the next attention
                kvb.kv_attn_decode(kvs[layer], q, t, k_new=kn, v_new=vn, log_beta_new=lb,
                                   num_splits=P, out=out, lse=lse, ws=ws_a, stream=main)
                attended[layer].record(main)
                side.wait_event(attended[layer])
                kvb.kv_evict_plan(kvs[layer], t, M, evicted_pos=evl, n_evicted=nev[layer],
                                  ws=ws_e[layer], stream=side)
                kvb.kv_evict_apply(kvs[layer], M, ws_e[layer], stream=side)
                continue
            kvb.kv_append(kvs[layer], kn, vn, lb, t, ws=ws_a, stream=main)
            appended[layer].record(main)
            side.wait_event(appended[layer])
            kvb.kv_evict_plan(kvs[layer], t, M, evicted_pos=evl, n_evicted=nev[layer],
                              ws=ws_e[layer], stream=side)
            kvb.kv_attn_decode(kvs[layer], q, t, num_splits=P, out=out, lse=lse, ws=ws_a,
                               stream=main)
            if deferred:
                planned[layer].record(side)
                continue
            attended[layer].record(main)
            side.wait_event(attended[layer])
            kvb.kv_evict_apply(kvs[layer], M, ws_e[layer], stream=side)
        if deferred:
            for layer in range(L):
                main.wait_event(planned[layer])
                kvb.kv_evict_apply(kvs[layer], M, ws_e[layer], stream=main)
        main.wait_stream(side)
        t.add_(1)

    # CPU baseline inputs: the whole heads of layer 0 as drawn (M tokens each, t = M)
    host_units = []
    if not args.no_cpu:
        import numpy as np
        torch.cuda.synchronize()
        d0, (q0, kn0, vn0, lb0) = kvs[0], qs[0]
        q0, kn0, vn0, lb0 = (x.cpu() for x in (q0, kn0, vn0, lb0))
        bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
        for u in range(w.units):
            b, g = divmod(u, w.hkv)
            host_units.append((0, b, g, bits(d0.k[b, g, :M + 1]), bits(d0.v[b, g, :M + 1]),
                               d0.log_beta[b, g, :M + 1].cpu().numpy(),
                               d0.pos[b, g, :M + 1].cpu().numpy(), M,
                               bits(q0[b, g * w.group:(g + 1) * w.group]), bits(kn0[b, g]),
                               bits(vn0[b, g]), float(lb0[b, g])))

    for _ in range(args.warmup + 1):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    replay_check = None
    if not args.no_cpu:
        replay_check = steady_replay_check(w, kvs[L - 1], qs[L - 1], t, out, lse, g, M, fill)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    nsteps = args.steps
    e0.record()
    for _ in range(nsteps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / nsteps
    assert bool((nev == 1).all()), "steady state: one eviction per head and layer"
    # eager steps with the kernel trace
    kvb.trace_enable(16 * L * args.steps + 64, ("attn_split", "attn_merge", "append",
                                                "evict_select", "compact_move", "evict_one",
                                                "one_shift"))
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    per = {}
    for name, kms in kvb.trace_read(1 << 20):
        per.setdefault(name, []).append(kms)
    kvb.trace_disable()
    split = {k: round(sum(v) / len(v) * 1000, 1) for k, v in per.items()}
    n = M + 1
    attn_b = algorithmic_bytes(w, n, 0)[0]

    # rows one step moves: each head's evicted slot e (from its evicted position and
    # the head's positions in order) moves min(e, n - 1 - e) rows with a start array
    # (the shorter side), n - 1 - e without; taken on one more eager step
    import numpy as np
    torch.cuda.synchronize()
    logical = []
    for c in kvs:
        pos_h = c.pos.cpu().numpy()
        st_h = c.start.cpu().numpy() if c.start is not None else np.zeros((B, w.hkv), np.int64)
        ln_h = c.length.cpu().numpy()
        logical.append((pos_h, st_h, ln_h))
    ev = torch.full((L, B, w.hkv, 1), -1, dtype=torch.int32, device="cuda")
    step(ev)
    torch.cuda.synchronize()
    evh = ev.cpu().numpy()
    moved = 0
    for layer, (pos_h, st_h, ln_h) in enumerate(logical):
        cap = pos_h.shape[2]
        if fill:
            # the decode token (position t - 1 of that step) moves into the evicted
            # slot unless it is the evicted token itself
            moved += int(np.sum(evh[layer, :, :, 0] != int(t[0].item()) - 1))
            continue
        for b in range(B):
            for g in range(w.hkv):
                nn = int(ln_h[b, g]) + 1                        # after the append
                order = (int(st_h[b, g]) + np.arange(nn - 1)) % cap
                p_log = np.append(pos_h[b, g, order], int(t[0].item()) - 1)
                e = int(np.searchsorted(p_log, evh[layer, b, g, 0]))
                moved += min(e, nn - 1 - e) if use_start else nn - 1 - e
    moves_b = algorithmic_bytes(w, n, moved)[1]
    step_b = L * attn_b + moves_b
    gbps = step_b / (ms * 1e-3) / 1e9
    attn_us = split.get("attn_split", 0.0)
    line = {
        "metric": "steady-state bounded-KV decode steps/s (evict 1 of M+1 per layer and step)",
        "value": round(1000.0 / ms, 3), "unit": "decode steps/s", "n_gpus": 1,
        "steps": nsteps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.head_dim, "budget": M, "layers": L, "graph": True,
                   "schedule": args.schedule or "fill",
                   "layout": "fill (evicted slot takes the decode token)" if fill
                   else "position order (shift)",
                   "head_start": use_start, "kv_splits": P},
        "eager_ms_per_step": round(eager_ms, 4), "kernel_us_eager": split,
        "attention_bytes_per_layer": attn_b, "moved_rows_per_step": moved,
        "bytes_per_step": step_b, "kv_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "attn_split_pipe128<G=4>" +
                     (" with eviction candidates" if plan1 or fill else "") +
                     " (M + 1 tokens)",
                     "achieved": round(attn_b / (attn_us * 1e-6) / 1e9, 1) if attn_us else None,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_b / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                     if attn_us else None,
                     "traffic": recorded_traffic(STEADY_TRAFFIC_FILE, splits=P, fill=fill,
                                                 head_start=use_start),
                     "bytes_per_launch": attn_b,
                     "avg_launch_ms": round(attn_us / 1000, 5)},
        "cpu_baseline": None}
    if host_units:
        line["cpu_baseline"] = cpu_baseline(w, host_units, M, M, args.cpu_seconds)
        line["cpu_baseline"]["checked_against_gpu"] = replay_check
    print(json.dumps(line), flush=True)


def steady_replay_check(w, c, qd, t, out, lse, graph, M, fill):
    """One replay of the captured steady step, checked against the oracle on its last
    layer (which the step's out and lse hold): that layer's heads are copied to the
    host before the replay; after it, every query head's out and lse must be within
    2e-3 of the oracle's (append, attend) and every head's live rows, in position
    order, equal bit for bit to the oracle's layout after the eviction."""
    import numpy as np
    import torch

    import oracle
    bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    torch.cuda.synchronize()
    q, kn, vn, lb = qd
    tq = int(t[0].item())
    B, H, G = w.batch, w.hkv, w.group

    def live(cc):
        k, v = bits(cc.k), bits(cc.v)
        lbh, ps, ln = cc.log_beta.cpu().numpy(), cc.pos.cpu().numpy(), cc.length.cpu().numpy()
        st = cc.start.cpu().numpy() if cc.start is not None else np.zeros((B, H), np.int64)
        cap = k.shape[2]
        rows = {}
        for b in range(B):
            for g in range(H):
                n = int(ln[b, g])
                sl = (int(st[b, g]) + np.arange(n)) % cap
                order = np.argsort(ps[b, g, sl], kind="stable")
                sl = sl[order]
                rows[(b, g)] = (k[b, g, sl], v[b, g, sl], lbh[b, g, sl], ps[b, g, sl], n)
        return rows

    before = live(c)
    qh, knh, vnh, lbh = bits(q), bits(kn), bits(vn), lb.cpu().numpy()
    graph.replay()
    torch.cuda.synchronize()
    after = live(c)
    oh, lh = out.cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for (b, g), (k, v, lbv, ps, n) in before.items():
        pad = lambda x: np.concatenate([x, np.zeros_like(x[:1])])[None, None]  # noqa: E731
        cc = oracle.Cache(pad(k), pad(v), pad(lbv), pad(ps), np.array([[n]], np.int32))
        oracle.append_tokens(cc, knh[b, g][None, None], vnh[b, g][None, None],
                             np.array([[lbh[b, g]]], np.float32), np.array([tq]))
        qv = (qh[b, g * G:(g + 1) * G].astype(np.uint32) << 16).view(np.float32)
        ro, rl = oracle.decode_attention(cc.values("k"), cc.values("v"), cc.log_beta, cc.pos,
                                         cc.length, qv.astype(np.float64)[None],
                                         np.array([tq]))
        for j in range(G):
            err = float(np.max(np.abs(oh[b, g * G + j] - ro[0, j])) / np.max(np.abs(ro[0, j])))
            assert err <= 2e-3 and abs(float(lh[b, g * G + j]) - rl[0, j]) <= 2e-3, \
                f"steady replay: query head ({b},{g * G + j}) rel err {err:.2e}"
            worst = max(worst, err)
        ce, _, _ = oracle.evict_to_budget(cc, np.array([tq]), M)
        kept = int(ce.length[0, 0])
        ka, va, la, pa, na = after[(b, g)]
        assert na == kept, f"steady replay: head ({b},{g}) len {na} vs {kept}"
        for got, name in ((ka, "k"), (va, "v"), (la, "log_beta"), (pa, "pos")):
            want = getattr(ce, name)[0, 0, :kept]
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), \
                f"steady replay: head ({b},{g}) {name} differs from the oracle"
    return {"what": "one replay of the captured step: the last layer's out/lse within 2e-3 "
                    "of the oracle (append, attend) and every head's live rows, in position "
                    "order, equal to the oracle's layout after the eviction",
            "kv_heads": len(before), "max_rel_err": float(f"{worst:.3e}"),
            "layout": "fill" if fill else "shift"}


def asm_bench(args):
    """Lookup + merge for one layer of the ASM workload's queries (32 sequences x 32
    query heads, 8 KV heads, D = 128): the linear scan and the two-level index
    (first-level clusters, top 16 kept), at 4K / 16K / 64K entries per KV head.
    Inputs are resident on the device; each figure is the mean of 50 back-to-back
    calls, and the per-kernel split comes from the library's HIP-event trace."""
    import dataclasses

    import numpy as np
    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    base = synth.WORKLOADS["asm_hier"]
    rows = []
    for K, K1 in ((4096, 64), (16384, synth.HIER_K1), (65536, 256)):
        w = dataclasses.replace(base, codebook=K)
        c1, offs, st, kid, ab, lz, cent = synth.host_hier_codebook(w, K, K1)
        q = synth.host_near_queries(w, cent)
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed)
        so = torch.randn((w.batch, w.hq, w.head_dim), device="cuda", generator=g)
        sl = torch.rand((w.batch, w.hq), device="cuda", generator=g) * 10
        dq, dc1, doffs, dst, dkid, dab, dlz, dcent = map(dev, (q, c1, offs, st, kid, ab, lz, cent))
        wsl = torch.empty(kvb.asm_lookup_merge_workspace(w.batch, w.hq, w.hkv, w.head_dim, K),
                          dtype=torch.uint8, device="cuda")
        wsh = torch.empty(kvb.asm_lookup_merge_hier_workspace(w.batch, w.hq, w.hkv, K1,
                                                              synth.HIER_M),
                          dtype=torch.uint8, device="cuda")
        calls = {
            "linear": lambda: kvb.asm_lookup_merge(dq, dcent, dab, dlz, so, sl, ws=wsl),
            "two_level": lambda: kvb.asm_lookup_merge_hier(dq, dc1, doffs, dst, dkid, synth.HIER_M,
                                                           dab, dlz, so, sl, ws=wsh),
        }
        row = {"entries": K, "clusters": K1, "kept": synth.HIER_M}
        idx = {}
        for name, fn in calls.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(50):
                _, _, i = fn()
            e1.record()
            torch.cuda.synchronize()
            kvb.trace_enable(16, ("asm_lookup", "asm_finalize"))
            fn()
            kern = [round(ms * 1000, 1) for _, ms in kvb.trace_read()]
            kvb.trace_disable()
            row[name + "_us"] = round(e0.elapsed_time(e1) / 50 * 1000, 2)
            row[name + "_kernels_us"] = kern
            idx[name] = i.cpu().numpy()
        row["same_index_fraction"] = float((idx["linear"] == idx["two_level"]).mean())
        rows.append(row)
        print(f"# {row}", file=sys.stderr, flush=True)
    mid = rows[1]
    print(json.dumps({
        "metric": "ASM lookup + merge latency per layer (two-level index, 16K entries)",
        "value": mid["two_level_us"], "unit": "us", "n_gpus": 1, "higher_is_better": False,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "asm_hier", "batch": base.batch, "q_heads": base.hq,
                   "kv_heads": base.hkv, "head_dim": base.head_dim},
        "sizes": rows}), flush=True)


def asm_step_bench(args):
    """One decode step of the ASM workload over its 36 layers: per layer, attention
    over the 2048 generated tokens of each (sequence, KV head) with the decode token
    appended (no retention bias), then the cosine lookup of every query head in its
    KV head's 4096-entry codebook and the merge of the chosen entry's state with the
    attention state -- by kv_attn_decode_asm (three launches), or with
    --asm-two-calls by kv_attn_decode then asm_lookup_merge (four).  Batch 32, 32 query / 8 KV heads, D = 128, bf16.  The caches
    and codebooks of all layers are resident; each step restores the lengths
    (untimed).  The attention kernel and the lookup are traced with HIP events on
    their stream in the timed steps."""
    import dataclasses

    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS["asm_lookup"]
    if args.layers:
        w = dataclasses.replace(w, layers=args.layers)
    L, B = w.layers, w.batch
    print(f"# generating {L} layers of {w.name}", file=sys.stderr, flush=True)
    caches, kvs, qs, books = [], [], [], []
    for layer in range(L):
        d = synth.device_cache(w, layer)
        caches.append(d)
        kvs.append(kvb.KVCache.from_dict(d))
        qs.append(synth.device_queries(w, layer))
        books.append(synth.device_codebook(w, layer))
    torch.cuda.synchronize()
    t = torch.full((B,), w.ctx, dtype=torch.int32, device="cuda")
    P = args.splits
    ws_a = torch.empty(kvb.kv_attn_decode_workspace(kvs[0], w.hq, P), dtype=torch.uint8,
                       device="cuda")
    ws_l = torch.empty(kvb.asm_lookup_merge_workspace(B, w.hq, w.hkv, w.head_dim, w.codebook),
                       dtype=torch.uint8, device="cuda")
    so = torch.empty((B, w.hq, w.head_dim), dtype=torch.float32, device="cuda")
    sl = torch.empty((B, w.hq), dtype=torch.float32, device="cuda")
    out = torch.empty_like(so)
    out_lse = torch.empty_like(sl)
    idx = torch.empty((B, w.hq), dtype=torch.int32, device="cuda")

    ws_f = torch.empty(kvb.kv_attn_decode_asm_workspace(kvs[0], w.hq, P, w.codebook),
                       dtype=torch.uint8, device="cuda")
    two_calls = args.asm_two_calls

    def step():
        for layer in range(L):
            q, kn, vn, _ = qs[layer]
            cent, abar, lz = books[layer]
            if two_calls:
                kvb.kv_attn_decode(kvs[layer], q, t, k_new=kn, v_new=vn, num_splits=P, out=so,
                                   lse=sl, ws=ws_a)
                kvb.asm_lookup_merge(q, cent, abar, lz, so, sl, out=out, out_lse=out_lse,
                                     idx=idx, ws=ws_l)
            else:
                kvb.kv_attn_decode_asm(kvs[layer], q, t, cent, abar, lz, k_new=kn, v_new=vn,
                                       num_splits=P, out=out, lse=out_lse, idx=idx, ws=ws_f)

    def restore():
        for d in caches:
            d["len"].fill_(w.ctx)

    # CPU baseline inputs: the whole KV heads of layer 0 with their codebooks
    host_units = []
    if not args.no_cpu:
        import numpy as np
        bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
        d0, (q0, kn0, vn0, _) = caches[0], qs[0]
        cent0, abar0, lz0 = books[0]
        cb = [(bits(cent0[g]), bits(abar0[g]), lz0[g].cpu().numpy()) for g in range(w.hkv)]
        for u in range(w.units):
            b, g = divmod(u, w.hkv)
            host_units.append((bits(d0["k"][b, g, :w.ctx + 1]), bits(d0["v"][b, g, :w.ctx + 1]),
                               d0["pos"][b, g, :w.ctx + 1].cpu().numpy(),
                               bits(q0[b, g * w.group:(g + 1) * w.group]), bits(kn0[b, g]),
                               bits(vn0[b, g]), cb[g]))

    for _ in range(args.warmup):
        restore()
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        restore()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            restore()
            graph.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        out_t = []
        for _ in range(args.steps):
            restore()
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out_t.append(e0.elapsed_time(e1))
        return out_t

    # the timed steps carry no trace events; kernel times come from further eager steps
    times = timed(graph.replay if graph is not None else step)
    kvb.trace_enable(4 * args.steps * L + 16, ("attn_split", "attn_merge", "asm_lookup",
                                               "asm_finalize"))
    timed(step)
    per = {}
    for name, kms in kvb.trace_read(1 << 16):
        per.setdefault(name, []).append(kms)
    kvb.trace_disable()
    ms = sum(times) / len(times)
    n = w.ctx + 1
    attn_b = algorithmic_bytes(w, n, 0)[0] - w.units * n * 8  # no bias: K, V, q, out only
    # the codebook, the chosen entry's state (bf16 a-bar row + log Z-bar) gathered per
    # query head, the chosen index written; q is read and (out, lse) written once, in
    # attn_b; the attention's own (out, lse) handed to a second call is overhead
    look_b = (w.hkv * w.codebook * w.head_dim * 2 + B * w.hq * (w.head_dim * 2 + 4)
              + B * w.hq * 4)
    split_ms = sum(per["attn_split"]) / len(per["attn_split"])
    # the split launch also scans the codebook (kv_attn_decode_asm): its bytes are the
    # attention's plus the codebook's
    unit_b = attn_b + (0 if two_calls else w.hkv * w.codebook * w.head_dim * 2)
    line = {
        "metric": "ASM decode steps/s (attention over 2048 tokens + centroid lookup + merge, "
                  "36 layers)",
        "value": round(1000.0 / ms, 3), "unit": "decode steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.head_dim, "tokens": w.ctx, "codebook": w.codebook,
                   "layers": L, "entry": "kv_attn_decode + asm_lookup_merge" if two_calls
                   else "kv_attn_decode_asm", "launch": "graph" if graph is not None
                   else "eager", "kv_splits": P or (
                       kvb.kv_attn_decode_splits(kvs[0], w.hq) if two_calls
                       else kvb.kv_attn_decode_asm_splits(kvs[0], w.hq, w.codebook))},
        "bytes_per_step": L * (attn_b + look_b),
        "gbps": round(L * (attn_b + look_b) / (ms * 1e-3) / 1e9, 1),
        "attn_split_us": round(split_ms * 1000, 2),
        "attn_split_gbps": round(attn_b / (split_ms * 1e-3) / 1e9, 1),
        "lookup_kernels_us": {k: round(sum(v) / len(v) * 1000, 2) for k, v in per.items()
                              if k != "attn_split"},
        "hbm_frac": round(L * (attn_b + look_b) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "attn_split_asm<G=4>" if not two_calls
                     else "attn_split_pipe128<G=4>",
                     "achieved": round(unit_b / (split_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(unit_b / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": unit_b,
                     "avg_launch_ms": round(split_ms, 5)},
        "cpu_baseline": asm_cpu_baseline(w, host_units, args.cpu_seconds) if host_units
        else None}
    print(json.dumps(line), flush=True)


def asm_cpu_baseline(w, host_units, budget_s):
    """The float64 oracle, as it stands, on whole KV heads of the ASM workload: append
    the decode token, attention of the head's query group over its 2049 tokens,
    cosine lookup of each query in the head's codebook and the merge; heads taken
    in turn until ``budget_s`` of CPU work; extrapolated to units x layers."""
    import numpy as np

    import oracle
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    f64 = lambda x: (np.asarray(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    done, elapsed = 0, 0.0
    for (k, v, pos, q, kn, vn, (cent, abar, lz)) in itertools.cycle(host_units):
        t0 = time.perf_counter()
        n = w.ctx
        c = oracle.Cache(k[None, None].copy(), v[None, None].copy(), None, pos[None, None].copy(),
                         np.array([[n]], np.int32))
        oracle.append_tokens(c, kn[None, None], vn[None, None], None, np.array([n]))
        so, sl = oracle.decode_attention(c.values("k"), c.values("v"), None, c.pos, c.length,
                                         f64(q)[None], np.array([n]))
        oracle.asm_lookup_merge(f64(q)[None], f64(cent)[None], f64(abar)[None],
                                np.asarray(lz, np.float64)[None], so, sl)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= budget_s:
            break
    step_s = elapsed / done * w.units * w.layers
    return {"value": 1.0 / step_s, "unit": "decode steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} runs over the {len(host_units)} whole KV heads of layer 0 "
                      f"({w.ctx + 1} tokens, {w.group} query heads, {w.codebook} codebook "
                      f"entries each: append + attention + lookup + merge), {elapsed:.1f} s, "
                      f"extrapolated to {w.units} heads x {w.layers} layers",
            "affinity_cpus": len(os.sched_getaffinity(0))}


def build_bench(args):
    """Offline build of one layer's attention-state memory (8 KV heads; per head
    16,384 calibration queries, a 16,384-token prefix encoded in 4 chunks, K-means
    into 4,096 entries for 10 iterations from 4,096 of the queries, then
    aggregation of the states).  Inputs are resident on the device; a step is one
    asm_build_memory call (the initial centroids are copied in first, a 16 MB
    device copy).  Kernel split and the MFMA roofline come from the library's
    HIP-event trace of one traced step."""
    import numpy as np
    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS["asm_build"]
    H, N, L, D, K = w.hkv, synth.BUILD_N, w.ctx, w.head_dim, w.codebook
    C, iters = synth.BUILD_CHUNKS, synth.BUILD_ITERS
    q, k, v = synth.host_asm_build(w, N)
    init = synth.host_kmeans_init(w, q, K)

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    dq, dk, dv, dinit = map(dev, (q, k, v, init))
    cent = torch.empty_like(dinit)
    cb = torch.empty((H, K, D), dtype=torch.bfloat16, device="cuda")
    ab = torch.empty((H, K, D), dtype=torch.bfloat16, device="cuda")
    lz = torch.empty((H, K), dtype=torch.float32, device="cuda")
    asg = torch.empty((H, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(kvb.asm_build_memory_workspace(H, N, D, L, C, K), dtype=torch.uint8,
                     device="cuda")

    def step():
        cent.copy_(dinit)
        kvb.asm_build_memory(dq, dk, dv, cent, iters, chunks=C, centroids_bf16=cb, abar=ab,
                             log_zbar=lz, assign=asg, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    names = ("asm_vt", "asm_prefix", "asm_prefix_merge", "km_assign", "km_update",
             "asm_aggregate")
    kvb.trace_enable(64, names)
    step()
    split = {}
    for name, t in kvb.trace_read():
        tot, n = split.get(name, (0.0, 0))
        split[name] = (tot + t, n + 1)
    kvb.trace_disable()
    flops = {"asm_prefix": 4.0 * H * N * L * D,          # S = QK^T and O = PV, per launch
             "km_assign": 2.0 * H * N * K * D}           # X C^T, per launch
    kern = {}
    for name, (tot, n) in split.items():
        row = {"launches": n, "total_ms": round(tot, 4), "avg_ms": round(tot / n, 4)}
        if name in flops:
            row["tflops"] = round(flops[name] / (tot / n * 1e-3) / 1e12, 1)
        kern[name] = row
    dom = max(flops, key=lambda nm: split.get(nm, (0.0, 1))[0])
    tot, n = split[dom]
    ach = flops[dom] / (tot / n * 1e-3) / 1e12
    print(f"# kernels {kern}", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "ASM memory build time per layer (prefix states, K-means, aggregation)",
        "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "asm_build", "kv_heads": H, "head_dim": D, "queries": N,
                   "prefix": L, "chunks": C, "entries": K, "iters": iters},
        "kernels": kern,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1),
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": round(ach / 2500.0, 4),
                     "traffic": None},
    }), flush=True)


def memento_bench(args):
    """MEMENTO-style erasure on the 1M-slot workload (batch 1, 64 query / 8 KV heads,
    D = 128, bf16; thinking blocks of 2K-16K tokens each followed by a 200-token
    memento): erase every completed block (range compaction), append the decode
    token and attend with beta == 1 over the kept tokens, evict to M = 65536 (a
    no-op).  Each trial restores the overwritten slots and the lengths first
    (untimed); the median over the trials is reported with min and max.  The calls
    are queued behind a GPU spin, so the times are device times."""
    import numpy as np
    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS["memento_1m"]
    blocks, ranges = synth.memento_layout(total=w.ctx, seed=w.seed)
    kept = 200 * (len(blocks) - 1) + blocks[-1][1]
    print(f"# memento_1m: {len(blocks)} blocks, {ranges.shape[0]} erased ranges, "
          f"{kept} tokens kept per KV head", file=sys.stderr, flush=True)
    dc = synth.device_cache(w, layer=0)
    q, kn, vn, _ = synth.device_queries(w, 0)
    c = kvb.KVCache.from_dict(dc)
    keep_slots = ((kept + 1 + 1023) // 1024) * 1024  # slots a trial overwrites
    prist = {k: dc[k][:, :, :keep_slots].clone() for k in ("k", "v", "pos")}
    rg = torch.from_numpy(ranges[None].copy()).cuda()
    nr = torch.tensor([ranges.shape[0]], dtype=torch.int32, device="cuda")
    t = torch.full((1,), w.ctx, dtype=torch.int32, device="cuda")
    ws_er = torch.empty(kvb.kv_erase_workspace(c), dtype=torch.uint8, device="cuda")
    # the caller knows the live length after the erase: split count by the library's
    # rule applied to it (about 2048 / (B * Hkv) splits, at most one per 256 live
    # slots) instead of to the 1M-slot capacity (512 splits)
    P_att = max(1, min(2048 // w.units, (kept + 1) // 256))
    if args.splits > 0:
        P_att = args.splits
    ws_a = torch.empty(kvb.kv_attn_decode_workspace(c, w.hq, P_att), dtype=torch.uint8,
                       device="cuda")
    ws_ev = torch.empty(kvb.kv_evict_workspace(c, w.budget), dtype=torch.uint8, device="cuda")
    n_er = torch.empty((1, w.hkv), dtype=torch.int32, device="cuda")
    n_ev = torch.empty((1, w.hkv), dtype=torch.int32, device="cuda")
    out = torch.empty((1, w.hq, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, w.hq), dtype=torch.float32, device="cuda")

    # a one-layer trial re-reads the same ~0.1-0.2 GB, which the 256 MB last-level
    # cache would otherwise keep between trials: 512 MB are written (untimed) before
    # each trial, so every trial starts from HBM as a layer of a real step would
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def restore():
        for k in ("k", "v", "pos"):
            dc[k][:, :, :keep_slots].copy_(prist[k])
        dc["len"].fill_(w.ctx)
        flush.fill_(1)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def trial():
        restore()
        torch.cuda.synchronize()
        # keep the GPU busy while the three calls are queued, so that the events
        # time the device work and not the host's launch latency
        torch.cuda._sleep(2_000_000)
        ev[0].record()
        kvb.kv_erase_ranges(c, rg, nr, n_erased=n_er, ws=ws_er)
        ev[1].record()
        kvb.kv_attn_decode(c, q, t, k_new=kn, v_new=vn, num_splits=P_att, out=out, lse=lse,
                           ws=ws_a)
        ev[2].record()
        kvb.kv_evict_to_budget(c, t, w.budget, n_evicted=n_ev, ws=ws_ev)
        ev[3].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(3)]

    for _ in range(args.warmup):
        trial()
    trials = max(args.steps, 20)
    res = np.array([trial() for _ in range(trials)])
    assert int(n_er.min()) == int(n_er.max()) == w.ctx - kept, "erased count"
    assert bool((dc["len"] == kept + 1).all()), "kept + decode token"
    assert int(n_ev.max()) == 0, "eviction to 65536 is a no-op"
    kvb.trace_enable(64 * trials + 64, ("erase_search", "erase_plan", "keep_count",
                                        "keep_emit", "compact_move", "attn_split",
                                        "attn_merge", "evict_select"))
    for _ in range(trials):
        trial()
    per = {}
    for name, kms in kvb.trace_read(1 << 16):
        per.setdefault(name, []).append(kms * 1000.0)
    kvb.trace_disable()
    U, D, e = w.units, w.head_dim, w.elem_bytes
    # kept rows moved (K, V, pos read and written); the erase locates each range's
    # slots by searching the sorted positions, so it reads no position scan
    erase_b = U * kept * 2 * (2 * D * e + 4)
    attn_b = algorithmic_bytes(w, kept + 1, 0)[0]
    med = np.median(res, axis=0)
    total = float(np.sum(med))
    print(json.dumps({
        "metric": "MEMENTO erase + bounded decode attention latency, one layer (1M-slot cache)",
        "value": round(total, 2), "unit": "us", "n_gpus": 1, "trials": trials,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": 1, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": D, "slots": w.ctx, "blocks": len(blocks),
                   "erased_ranges": int(ranges.shape[0]), "kept": kept, "budget": w.budget,
                   "attention_splits": P_att},
        "erase_us": {"median": round(float(med[0]), 2), "min": round(float(res[:, 0].min()), 2),
                     "max": round(float(res[:, 0].max()), 2),
                     "bytes": erase_b, "gbps": round(erase_b / (med[0] * 1e-6) / 1e9, 1)},
        "attention_us": {"median": round(float(med[1]), 2), "min": round(float(res[:, 1].min()), 2),
                         "max": round(float(res[:, 1].max()), 2),
                         "bytes": attn_b, "gbps": round(attn_b / (med[1] * 1e-6) / 1e9, 1)},
        "evict_us": {"median": round(float(med[2]), 2)},
        "kernel_us": {k: round(float(np.median(v)), 1) for k, v in per.items()}}), flush=True)


def memento_paged_bench(args):
    """The MEMENTO trial of memento_bench over a paged cache: the same 1M-token trace
    laid out in 32-slot pages, every thinking block and every memento starting on a
    fresh page (its last page partly filled; physical pages in a seeded random
    order).  The erase drops the completed blocks' pages from each head's page table
    (no row moves); the decode token goes into the last page (or a free page) and
    the attention reads the kept pages.  Each trial restores the page arrays and
    the lengths first (untimed); median over the trials, device times."""
    import numpy as np
    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS["memento_1m"]
    blocks, ranges = synth.memento_layout(total=w.ctx, seed=w.seed)
    full = args.full_pages
    if full:
        # the trace in full pages: blocks end inside pages, so each erased range
        # leaves a partly erased page at both ends (compacted in place)
        n = w.ctx // 32
        phys = n + 64
        prng = np.random.Generator(np.random.PCG64(w.seed + 77))
        table = np.stack([prng.permutation(phys)[:n] for _ in range(w.hkv)]).astype(np.int32)
        fill = np.full(n, 32, np.int32)
        pos0 = (32 * np.arange(n)).astype(np.int32)
        # a page stays unless one range holds all its 32 positions
        j = np.searchsorted(ranges[:, 0], pos0, side="right") - 1
        inside = (j >= 0) & (ranges[np.maximum(j, 0), 1] >= pos0 + 32)
        keep = np.nonzero(~inside)[0]
        kept = 200 * (len(blocks) - 1) + blocks[-1][1]
        tok = np.arange(w.ctx)
        jt = np.searchsorted(ranges[:, 0], tok, side="right") - 1
        gone = ((jt >= 0) & (tok < ranges[np.maximum(jt, 0), 1])).reshape(n, 32)
        n_partial = int((gone.any(axis=1) & ~gone.all(axis=1)).sum())
    else:
        table, fill, pos0, phys = synth.memento_pages(blocks, w.hkv, seed=w.seed)
        n = table.shape[1]
        n_partial = 0
        erased = np.zeros(n, bool)
        for s0, e0 in ranges:
            erased |= (pos0 >= s0) & (pos0 < e0)
        keep = np.nonzero(~erased)[0]
        kept = int(fill[keep].sum())
    print(f"# memento_1m paged: {len(blocks)} blocks, {n} pages ({phys} physical), "
          f"{keep.size} pages and {kept} tokens kept per KV head", file=sys.stderr, flush=True)
    cap = 32 * phys
    dc = synth.device_cache(w, layer=0, n=cap, cap=cap)
    pos = np.zeros((w.hkv, cap), np.int32)
    for g in range(w.hkv):
        for i in range(n):
            pos[g, 32 * table[g, i]:32 * table[g, i] + fill[i]] = pos0[i] + np.arange(fill[i])
    dc["pos"].copy_(torch.from_numpy(pos[None]))
    c = kvb.KVCache.from_dict(dc)
    # the rows a partly erased page moves, restored before each trial
    prist = {k: dc[k].clone() for k in ("k", "v", "pos")} if full else None
    mp = n + 8
    tab0 = np.full((1, w.hkv, mp), -1, np.int32)
    tab0[0, :, :n] = table
    fil0 = np.zeros((1, w.hkv, mp), np.int32)
    fil0[0, :, :n] = fill
    tab0, fil0 = torch.from_numpy(tab0).cuda(), torch.from_numpy(fil0).cuda()
    pg = kvb.KVPages(tab0.clone(), fil0.clone(),
                     torch.full((1, w.hkv), n, dtype=torch.int32, device="cuda"))
    free = [min(set(range(phys)) - set(table[g].tolist())) for g in range(w.hkv)]
    spare = torch.tensor([free], dtype=torch.int32, device="cuda")
    q, kn, vn, _ = synth.device_queries(w, 0)
    rg = torch.from_numpy(ranges[None].copy()).cuda()
    nr = torch.tensor([ranges.shape[0]], dtype=torch.int32, device="cuda")
    t = torch.full((1,), w.ctx, dtype=torch.int32, device="cuda")
    ws_er = torch.empty(kvb.kv_erase_paged_workspace(c, pg), dtype=torch.uint8, device="cuda")
    # split count by the library's rule applied to the pages left after the erase
    # (about 2048 / (B * Hkv) splits, at most one per 8 pages)
    P_att = max(1, min(2048 // w.units, (keep.size + 1) // 8))
    if args.splits > 0:
        P_att = args.splits
    ws_a = torch.empty(kvb.kv_attn_decode_workspace(c, w.hq, P_att), dtype=torch.uint8,
                       device="cuda")
    n_er = torch.empty((1, w.hkv), dtype=torch.int32, device="cuda")
    out = torch.empty((1, w.hq, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, w.hq), dtype=torch.float32, device="cuda")

    # every trial from HBM: 512 MB written (untimed) before each one, more than the
    # 256 MB last-level cache holds
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def restore():
        pg.table.copy_(tab0)
        pg.fill.copy_(fil0)
        pg.n_pages.fill_(n)
        dc["len"].fill_(int(fill.sum()))
        if prist is not None:
            for k in prist:
                dc[k].copy_(prist[k])
        flush.fill_(1)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def trial():
        restore()
        torch.cuda.synchronize()
        torch.cuda._sleep(2_000_000)
        ev[0].record()
        kvb.kv_erase_ranges_paged(c, pg, rg, nr, n_erased=n_er, ws=ws_er)
        ev[1].record()
        kvb.kv_attn_decode_paged(c, pg, q, t, k_new=kn, v_new=vn, spare=spare,
                                 num_splits=P_att, out=out, lse=lse, ws=ws_a)
        ev[2].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(2)]

    for _ in range(args.warmup):
        trial()
    trials = max(args.steps, 20)
    res = np.array([trial() for _ in range(trials)])
    assert int(n_er.min()) == int(n_er.max()) == w.ctx - kept, "erased count"
    assert bool((dc["len"] == kept + 1).all()), "kept + decode token"
    assert bool((pg.n_pages >= keep.size).all()), "pages kept"
    kvb.trace_enable(8 * trials + 64, ("erase_pages", "attn_split", "attn_merge"))
    for _ in range(trials):
        trial()
    per = {}
    for name, kms in kvb.trace_read(1 << 16):
        per.setdefault(name, []).append(kms * 1000.0)
    kvb.trace_disable()
    D = w.head_dim
    attn_b = algorithmic_bytes(w, kept + 1, 0)[0]
    med = np.median(res, axis=0)
    print(json.dumps({
        "metric": "MEMENTO erase + bounded decode attention latency, one layer (1M-token "
                  "paged cache)",
        "value": round(float(np.sum(med)), 2), "unit": "us", "n_gpus": 1, "trials": trials,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name,
                   "layout": ("paged (32-slot pages, full; blocks end inside pages)" if full
                              else "paged (32-slot pages, block-aligned)"),
                   "batch": 1, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": D,
                   "tokens": w.ctx, "pages": n, "pages_kept": int(keep.size),
                   "erased_ranges": int(ranges.shape[0]), "kept": kept,
                   "attention_splits": P_att},
        "erase_us": {"median": round(float(med[0]), 2), "min": round(float(res[:, 0].min()), 2),
                     "max": round(float(res[:, 0].max()), 2),
                     "partial_pages_per_head": n_partial},
        "attention_us": {"median": round(float(med[1]), 2), "min": round(float(res[:, 1].min()), 2),
                         "max": round(float(res[:, 1].max()), 2),
                         "bytes": attn_b, "gbps": round(attn_b / (med[1] * 1e-6) / 1e9, 1)},
        "kernel_us": {k: round(float(np.median(v)), 1) for k, v in per.items()}}), flush=True)


def paged_attn_bench(args):
    """The 32K workload's attention over a paged cache: each KV head's 32,768 tokens
    in 1024 full 32-slot pages placed on a seeded random permutation of 1032
    physical pages, against the same tokens laid out contiguously (gathered page by
    page on the device).  No decode token; the library's default split counts.
    Both outputs are compared (within 2e-3); mean time per call over repeated calls
    (HIP events, the calls queued behind a GPU spin)."""
    import numpy as np
    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS["qwen3_8b_32k"]
    n = w.ctx
    npg = n // 32
    phys = npg + 8
    cap = 32 * phys
    dc = synth.device_cache(w, layer=0, n=cap, cap=cap)
    rng = np.random.Generator(np.random.PCG64(w.seed + 91))
    table = np.stack([rng.permutation(phys)[:npg] for _ in range(w.units)]).astype(np.int32)
    tab = torch.from_numpy(table).cuda().view(w.batch, w.hkv, npg)
    # slot of logical token j: 32 * table[j / 32] + j % 32; positions = logical index
    slot = (tab.long()[..., :, None] * 32 + torch.arange(32, device="cuda")).reshape(
        w.batch, w.hkv, n)
    pos = torch.zeros((w.batch, w.hkv, cap), dtype=torch.int32, device="cuda")
    pos.scatter_(2, slot, torch.arange(n, dtype=torch.int32, device="cuda").expand(
        w.batch, w.hkv, n).contiguous())
    dc["pos"].copy_(pos)
    dc["len"].fill_(n)
    c = kvb.KVCache.from_dict(dc)
    pg = kvb.KVPages(tab.contiguous(), torch.full((w.batch, w.hkv, npg), 32, dtype=torch.int32,
                                                  device="cuda"),
                     torch.full((w.batch, w.hkv), npg, dtype=torch.int32, device="cuda"))
    # the same tokens contiguous, in logical order
    cont = {}
    for name in ("k", "v", "log_beta"):
        x = dc[name]
        if x is None:
            cont[name] = None
            continue
        idx = slot if x.dim() == 3 else slot[..., None].expand(-1, -1, -1, w.head_dim)
        cont[name] = torch.gather(x, 2, idx).contiguous()
    cont["pos"] = torch.arange(n, dtype=torch.int32, device="cuda").expand(
        w.batch, w.hkv, n).contiguous()
    cont["len"] = torch.full((w.batch, w.hkv), n, dtype=torch.int32, device="cuda")
    cc = kvb.KVCache.from_dict(cont)
    q, _, _, _ = synth.device_queries(w, 0)
    t = torch.full((w.batch,), n, dtype=torch.int32, device="cuda")
    ws_p = torch.empty(kvb.kv_attn_decode_workspace(c, w.hq, 0), dtype=torch.uint8,
                       device="cuda")
    ws_c = torch.empty(kvb.kv_attn_decode_workspace(cc, w.hq, 0), dtype=torch.uint8,
                       device="cuda")
    outs = {}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        torch.cuda._sleep(2_000_000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1000.0

    def run_paged():
        outs["p"] = kvb.kv_attn_decode_paged(c, pg, q, t, ws=ws_p)

    def run_cont():
        outs["c"] = kvb.kv_attn_decode(cc, q, t, ws=ws_c)

    reps = max(args.steps, 20)
    us_p = timed(run_paged, reps)
    us_c = timed(run_cont, reps)
    (op, lp), (oc, lc) = outs["p"], outs["c"]
    den = oc.abs().amax(dim=-1).clamp_min(1e-30)
    rel = float(((op - oc).abs().amax(dim=-1) / den).max())
    dl = float((lp - lc).abs().max())
    assert rel <= 2e-3 and dl <= 2e-3, (rel, dl)
    by = algorithmic_bytes(w, n, 0)[0]
    print(json.dumps({
        "metric": "paged vs contiguous decode attention, one layer of the 32K workload",
        "value": round(us_p, 2), "unit": "us", "n_gpus": 1, "reps": reps,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.head_dim, "tokens": n, "pages": npg, "physical_pages": phys},
        "paged": {"us": round(us_p, 2), "gbps": round(by / (us_p * 1e-6) / 1e9, 1),
                  "frac": round(by / (us_p * 1e-6) / 8e12, 4)},
        "contiguous": {"us": round(us_c, 2), "gbps": round(by / (us_c * 1e-6) / 1e9, 1),
                       "frac": round(by / (us_c * 1e-6) / 8e12, 4)},
        "bytes": by, "max_rel_err_vs_contiguous": rel, "max_lse_diff": dl}), flush=True)


def latent_bench(args):
    """Latent memory of evicted tokens, one layer of the 32K decode workload (batch
    16, 8 KV heads, D = 128): the update after the eviction of 32769 -> 4096 tokens
    per KV head (28,673 absorbed each), the update in the steady state (one token per
    KV head), and the read-out for the 32 query heads.  Plans are made once
    (neither call changes the cache); each figure is the mean of repeated calls."""
    import numpy as np
    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS["qwen3_8b_32k"]
    B, H, D, M = w.batch, w.hkv, w.head_dim, w.budget
    prm = synth.host_latent_params(D, w.hq, 77)
    mM = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    mb = torch.zeros((B, H, D), dtype=torch.float32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1000.0

    rows = {}
    for name, n in (("evict_32k", w.ctx + 1), ("steady", M + 1)):
        dc = synth.device_cache(w, layer=0, n=n, cap=n + 31)
        c = kvb.KVCache.from_dict(dc)
        t = torch.full((B,), n, dtype=torch.int32, device="cuda")
        nev, ws_e = kvb.kv_evict_plan(c, t, M)
        ws = torch.empty(kvb.kv_latent_absorb_workspace(c), dtype=torch.uint8, device="cuda")
        us = timed(lambda: kvb.kv_latent_absorb(c, M, ws_e, prm["lam"], mM, mb, ws=ws),
                   10 if name == "evict_32k" else 50)
        ne = int(nev.sum().item())
        # algorithmic bytes: the evicted rows read once, the state read and written
        byts = ne * 2 * D * 2 + 2 * B * H * (D * D + D) * 4
        rows[name] = {"evicted_per_head": ne // (B * H), "us": round(us, 1),
                      "bytes": byts, "gbps": round(byts / (us * 1e-6) / 1e9, 1),
                      "tflops": round(2.0 * ne * D * D / (us * 1e-6) / 1e12, 1)}
        print(f"# {name} {rows[name]}", file=sys.stderr, flush=True)
        del dc, c
        torch.cuda.empty_cache()
    q = synth.device_queries(w, 0)[0]
    out = torch.zeros((B, w.hq, D), dtype=torch.float32, device="cuda")
    W_o, w_g, c_g = (torch.from_numpy(prm[k]).cuda() for k in ("W_o", "w_g", "c_g"))
    mb.fill_(1.0)
    us = timed(lambda: kvb.kv_latent_read(q, mM, mb, W_o, w_g, c_g, prm["eps"], out), 50)
    rows["read"] = {"us": round(us, 1)}
    ev = rows["evict_32k"]
    print(json.dumps({
        "metric": "latent-memory update after evicting 32769 -> 4096 tokens per KV head",
        "value": ev["us"], "unit": "us", "n_gpus": 1, "higher_is_better": False,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3_8b_32k (one layer)", "batch": B, "kv_heads": H,
                   "head_dim": D, "budget": M, "lam": prm["lam"]},
        "roofline": {"bound": "hbm", "kernel": "latent_absorb_part + list + combine",
                     "achieved": ev["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ev["gbps"] / HBM_PEAK_GBPS, 4), "traffic": None},
        "cases": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3_8b_32k")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (testing)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--serial", action="store_true",
                    help="run each layer's eviction planning on the attention stream (no overlap)")
    ap.add_argument("--schedule", default=None,
                    choices=["plan_beside", "both_beside", "deferred", "deferred_plan",
                             "fused_append", "evict_one", "plan_one", "fill"],
                    help="deferred_plan (default of the 32K step): all layers' eviction "
                         "plans and compactions follow the last attention, each plan running "
                         "beside the previous layer's compaction; deferred: each plan beside "
                         "its layer's attention, the compactions after the last attention; "
                         "plan_beside: each compaction right after its layer's attention; "
                         "both_beside: each compaction beside the next layer's attention; "
                         "fused_append (--steady): the attention call appends, each layer's "
                         "plan and compaction beside the next layer's attention; evict_one "
                         "(--steady): the attention call appends, each layer's one-launch "
                         "eviction (kv_evict_one) beside the next layer's attention; fill "
                         "(--steady default): one kv_attn_decode_evict_one call per layer "
                         "(the decode token takes the evicted slot); plan_one (--steady): "
                         "kv_attn_decode_plan_one, each layer's order-keeping "
                         "kv_evict_one_apply beside the next layer's attention")
    ap.add_argument("--graph", action="store_true",
                    help="ASM step: replay the step as one captured HIP graph (the decode "
                         "step does so unless --eager)")
    ap.add_argument("--eager", action="store_true",
                    help="decode step: launch the step's kernels one by one instead of "
                         "replaying the step captured once as a HIP graph")
    ap.add_argument("--fused", action="store_true",
                    help="fused attention + compaction kernels (kv_attn_decode_compact) instead "
                         "of attention followed by a separate compaction pass")
    ap.add_argument("--no-start", action="store_true",
                    help="steady state: heads without a first-slot entry (every eviction "
                         "shifts the rows after the evicted slot)")
    ap.add_argument("--steady", action="store_true",
                    help="time the steady-state decode loop instead: every KV head holds M "
                         "tokens, each step appends one and evicts one (one JSON line)")
    ap.add_argument("--asm-lookup", action="store_true",
                    help="time the attention-state-memory lookup + merge instead: linear and "
                         "two-level index at 4K, 16K and 64K entries per KV head (one JSON line)")
    ap.add_argument("--asm-build", action="store_true",
                    help="time the offline build of one layer's attention-state memory "
                         "(prefix states in 4 chunks, K-means, aggregation; one JSON line)")
    ap.add_argument("--asm-step", action="store_true",
                    help="time one decode step of the ASM workload (36 layers of attention "
                         "over 2048 tokens + lookup + merge) instead (one JSON line)")
    ap.add_argument("--asm-two-calls", action="store_true",
                    help="--asm-step: attention and lookup + merge as two calls")
    ap.add_argument("--memento", action="store_true",
                    help="time MEMENTO erasure + attention on the 1M-slot workload instead "
                         "(one JSON line)")
    ap.add_argument("--paged", action="store_true",
                    help="--memento: the same trial over a paged cache (block-granular "
                         "erase, paged attention); alone: the 32K workload's attention "
                         "over a paged cache against the contiguous one (one JSON line)")
    ap.add_argument("--full-pages", action="store_true",
                    help="--memento --paged: the trace in full pages (blocks not aligned to "
                         "pages; the erase compacts partly erased pages)")
    ap.add_argument("--latent", action="store_true",
                    help="time the latent memory of evicted tokens (update after the 32K "
                         "eviction, steady-state update, read-out; one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy kernel 5 times (scales the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        y = torch.empty_like(x)
        for _ in range(5):
            torch.mul(x, 1.0, out=y)        # elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "elementwise copy", "bytes_read": 1 << 30,
                          "bytes_written": 1 << 30, "launches": 5}))
        return
    if args.asm_lookup:
        asm_bench(args)
        return
    if args.asm_build:
        build_bench(args)
        return
    if args.latent:
        latent_bench(args)
        return
    if args.memento and args.paged:
        memento_paged_bench(args)
        return
    if args.paged:
        paged_attn_bench(args)
        return
    if args.memento:
        memento_bench(args)
        return
    if args.asm_step:
        asm_step_bench(args)
        return
    if args.steady:
        steady_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(the hot path shards by KV head with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import numpy as np
    import torch

    import bounded_decode_attention_amd as kvb
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.layers:
        w = dataclasses.replace(w, layers=args.layers)
    L, M, B = w.layers, w.budget, w.batch
    n = w.ctx + 1
    dev = "cuda"
    print(f"# generating {L} layers of {w.name} on the device", file=sys.stderr, flush=True)
    caches, kvs, qs, prist = [], [], [], []
    for layer in range(L):
        d = synth.device_cache(w, layer)
        caches.append(d)
        kvs.append(kvb.KVCache.from_dict(d))
        qs.append(synth.device_queries(w, layer))
        prist.append({k: d[k][:, :, :M].clone() for k in ("k", "v", "log_beta", "pos")})
    torch.cuda.synchronize()
    t = torch.full((B,), w.ctx, dtype=torch.int32, device=dev)
    outs = [torch.empty((B, w.hq, w.head_dim), dtype=torch.float32, device=dev) for _ in range(L)]
    lses = [torch.empty((B, w.hq), dtype=torch.float32, device=dev) for _ in range(L)]
    nev = [torch.empty((B, w.hkv), dtype=torch.int32, device=dev) for _ in range(L)]
    first_ev = [torch.empty((B, w.hkv, 1), dtype=torch.int32, device=dev) for _ in range(L)]
    ws_a = torch.empty(kvb.kv_attn_decode_workspace(kvs[0], w.hq, args.splits), dtype=torch.uint8,
                       device=dev)
    sched = "serial" if args.serial else (args.schedule or "deferred_plan")
    if args.fused and sched in ("deferred", "deferred_plan"):
        # the fused pair needs the layer's plan between its two phases
        if args.schedule:
            sys.exit(f"bench.py: --fused needs the plan before each layer's second phase; "
                     f"--schedule {args.schedule} defers it")
        sched = "plan_beside"
    # one eviction workspace per layer when the plans outlive the next layer's planning;
    # zero-filled, so a plan header that was never written reads as 'nothing to do'
    n_ws = L if sched in ("deferred", "deferred_plan") else 1
    ws_es = [torch.zeros(kvb.kv_evict_workspace(kvs[0], M), dtype=torch.uint8, device=dev)
             for _ in range(n_ws)]
    splits = args.splits or kvb.kv_attn_decode_splits(kvs[0], w.hq)

    def restore():
        for d, p in zip(caches, prist):
            for k in ("k", "v", "log_beta", "pos"):
                d[k][:, :, :M].copy_(p[k])
            d["len"].fill_(w.ctx)

    # Per layer: append the decode token, plan the eviction (reads log beta and
    # positions only) on a side stream beside the attention over the whole cache,
    # then compact (re-reads the kept rows, writes them to their slots).  Where the
    # compaction runs is the schedule: after the last layer's attention (deferred,
    # the default: a layer is not attended again before the next step, and HBM sees
    # the step's reads and its writes in two phases instead of interleaved), right
    # after the layer's attention (plan_beside), or beside the next layer's
    # attention on the side stream (both_beside).  --fused: attention over the tiles below
    # the destination boundary runs beside the planner; the rest waits for the plan
    # and writes every kept row to its compacted slot from the data it has loaded.
    # Layer l+1's work starts after layer l's attention (its inputs would come from
    # it).  The side stream has default priority and is joined at the end.
    side_stream = torch.cuda.Stream()
    appended = [torch.cuda.Event() for _ in range(L)]
    planned = [torch.cuda.Event() for _ in range(L)]
    attended = [torch.cuda.Event() for _ in range(L)]
    fused = args.fused

    def step(main):
        side = main if sched == "serial" else side_stream
        for layer in range(L):
            q, kn, vn, lb = qs[layer]
            ws_e = ws_es[layer % n_ws]
            if sched != "deferred_plan":  # deferred_plan: the attention call appends
                kvb.kv_append(kvs[layer], kn, vn, lb, t, ws=ws_a, stream=main)
            if sched != "deferred_plan":
                if side is not main:
                    appended[layer].record(main)
                    side.wait_event(appended[layer])
                kvb.kv_evict_plan(kvs[layer], t, M, evicted_pos=first_ev[layer],
                                  n_evicted=nev[layer], ws=ws_e, stream=side)
            if fused:
                kvb.kv_attn_decode_compact(kvs[layer], q, t, M, ws_e, num_splits=args.splits,
                                           phase=1, out=outs[layer], lse=lses[layer], ws=ws_a,
                                           stream=main)
                if side is not main:
                    planned[layer].record(side)
                    main.wait_event(planned[layer])
                kvb.kv_attn_decode_compact(kvs[layer], q, t, M, ws_e, num_splits=args.splits,
                                           phase=2, out=outs[layer], lse=lses[layer], ws=ws_a,
                                           stream=main)
                continue
            if sched == "deferred_plan":
                kvb.kv_attn_decode(kvs[layer], q, t, k_new=kn, v_new=vn, log_beta_new=lb,
                                   num_splits=args.splits, out=outs[layer], lse=lses[layer],
                                   ws=ws_a, stream=main)
            else:
                kvb.kv_attn_decode(kvs[layer], q, t, num_splits=args.splits, out=outs[layer],
                                   lse=lses[layer], ws=ws_a, stream=main)
            if sched == "both_beside":
                attended[layer].record(main)
                side.wait_event(attended[layer])
                kvb.kv_evict_apply(kvs[layer], M, ws_e, stream=side)
            elif sched in ("plan_beside", "serial"):
                if side is not main:
                    planned[layer].record(side)
                    main.wait_event(planned[layer])
                kvb.kv_evict_apply(kvs[layer], M, ws_e, stream=main)
            elif sched == "deferred":
                planned[layer].record(side)
        if sched == "deferred_plan":
            attended[0].record(main)
            side.wait_event(attended[0])
            for layer in range(L):
                kvb.kv_evict_plan(kvs[layer], t, M, evicted_pos=first_ev[layer],
                                  n_evicted=nev[layer], ws=ws_es[layer], stream=side)
                planned[layer].record(side)
        if sched in ("deferred", "deferred_plan"):
            for layer in range(L):
                main.wait_event(planned[layer])
                kvb.kv_evict_apply(kvs[layer], M, ws_es[layer], stream=main)
        if side is not main:
            main.wait_stream(side)

    for _ in range(args.warmup):
        restore()
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        # the whole step (both streams) captured once; replayed after each restore
        restore()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            restore()
            graph.replay()
        torch.cuda.synchronize()

    # CPU baseline inputs: whole heads of layer 0 as drawn (read before the timed run)
    # (the first and the last layer: the last one's plan runs last in the default schedule)
    host_units = []
    if not args.no_cpu:
        restore()
        torch.cuda.synchronize()
        for layer in sorted({0, L - 1}):
            d0 = caches[layer]
            q0, kn0, vn0, lb0 = (x.cpu() for x in qs[layer])
            for u in range(w.units):
                b, g = divmod(u, w.hkv)
                host_units.append((
                    layer, b, g,
                    # slots 0 .. ctx (the append overwrites slot ctx)
                    d0["k"][b, g, :n].view(torch.int16).cpu().numpy().view(np.uint16),
                    d0["v"][b, g, :n].view(torch.int16).cpu().numpy().view(np.uint16),
                    d0["log_beta"][b, g, :n].cpu().numpy(),
                    d0["pos"][b, g, :n].cpu().numpy(), w.ctx,
                    q0[b, g * w.group:(g + 1) * w.group].view(torch.int16).numpy()
                    .view(np.uint16),
                    kn0[b, g].view(torch.int16).numpy().view(np.uint16),
                    vn0[b, g].view(torch.int16).numpy().view(np.uint16), float(lb0[b, g])))

    # secondary reference: a plain device copy (reads and writes 1 GiB each per call)
    cx = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cy = torch.empty_like(cx)
    cy.copy_(cx)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        cy.copy_(cx)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cx, cy

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    if graph is not None:
        for _ in range(args.steps):
            restore()
            torch.cuda.synchronize()
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
    kvb.trace_enable(2 * args.steps * L + 16, ("attn_split", "attn_fused"))
    eager_times = []
    for _ in range(args.steps):
        restore()
        torch.cuda.synchronize()
        e0.record()
        step(torch.cuda.current_stream())
        e1.record()
        torch.cuda.synchronize()
        eager_times.append(e0.elapsed_time(e1))
    if graph is None:
        times = eager_times
    trace = kvb.trace_read()
    kvb.trace_disable()
    # per layer: the attention split launch(es) of that layer (fused: both phases)
    split_ms = [ms for name, ms in trace if name == "attn_split"]
    fused_ms = [ms for name, ms in trace if name == "attn_fused"]

    # the timed step (graph replay, or eager) once more on restored inputs; its results
    # for the CPU baseline's layers are kept on the host and compared with the oracle's
    # in the cpu_baseline leg
    gpu_res = None
    if host_units:
        restore()
        torch.cuda.synchronize()
        if graph is not None:
            graph.replay()
        else:
            step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        gpu_res = {}
        for layer in sorted({hu[0] for hu in host_units}):
            d = caches[layer]
            gpu_res[layer] = {
                "out": outs[layer].cpu().numpy(), "lse": lses[layer].cpu().numpy(),
                "len": d["len"].cpu().numpy(),
                "k": d["k"][:, :, :M].view(torch.int16).cpu().numpy().view(np.uint16),
                "v": d["v"][:, :, :M].view(torch.int16).cpu().numpy().view(np.uint16),
                "log_beta": d["log_beta"][:, :, :M].cpu().numpy(),
                "pos": d["pos"][:, :, :M].cpu().numpy()}

    # sanity: every head evicted to M; moved rows from the first evicted position
    moved = 0
    for layer in range(L):
        assert bool((nev[layer] == n - M).all()), "eviction count"
        p0 = first_ev[layer].clamp(max=M).sum().item()
        moved += w.units * M - p0
    attn_b, move_b = algorithmic_bytes(w, n, 0)
    total_b = L * attn_b + algorithmic_bytes(w, n, moved)[1]
    ms_per_step = sum(times) / len(times)
    gbps = total_b / (ms_per_step * 1e-3) / 1e9
    if fused:
        # the fused pair reads every row once and writes the moved rows once
        assert len(split_ms) == len(fused_ms)
        unit_b = attn_b + (moved // L) * (2 * w.head_dim * w.elem_bytes + 8)
        pair = [a + b for a, b in zip(split_ms, fused_ms)]
        split_avg = sum(pair) / len(pair)
        kernel = "attn_split_pipe128<G=4> phases 1+2 (attention + compaction writes)"
    else:
        unit_b = attn_b
        split_avg = sum(split_ms) / len(split_ms)
        kernel = "attn_split_pipe128<G=4>"
    split_gbps = unit_b / (split_avg * 1e-3) / 1e9

    traffic = recorded_traffic(TRAFFIC_FILE, splits=splits, fused=fused)

    line = {
        "metric": METRIC, "value": round(1000.0 / ms_per_step, 3), "unit": "decode steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.head_dim, "ctx": w.ctx, "budget": M, "layers": L,
                   "kv_splits": splits,
                   "schedule": sched,
                   "compaction": "fused" if fused else "separate pass",
                   "launch": "graph" if graph is not None else "eager"},
        "kv_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "device_copy_gbps": round(copy_gbps, 1), "copy_frac": round(gbps / copy_gbps, 4),
        "bytes_per_step": total_b, "moved_rows_per_step": moved,
        "eager_ms_per_step": round(sum(eager_times) / len(eager_times), 4),
        # graph replays carry no events: kernel times come from the
        # eager steps that follow them (same kernels, same inputs)
        "kernel_times_from": "eager steps" if graph is not None else "timed steps",
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(split_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(split_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": unit_b, "avg_launch_ms": round(split_avg, 5),
                     "launches": len(split_ms)},
        "cpu_baseline": None,
    }
    if fused:
        line["roofline"]["phase_ms"] = [round(sum(split_ms) / len(split_ms), 5),
                                        round(sum(fused_ms) / len(fused_ms), 5)]
    if host_units:
        line["cpu_baseline"] = cpu_baseline(w, host_units, w.ctx, M, args.cpu_seconds,
                                            gpu_res)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
