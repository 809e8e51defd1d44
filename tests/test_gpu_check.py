"""kv_check_cache: each precondition violation, planted in otherwise valid caches
(every value in bounds), sets exactly its bit on exactly the affected heads."""
import numpy as np
import pytest
import torch

import bounded_decode_attention_amd as kvb
import synth
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu

BITS = kvb.CHECK_BITS


def _base(start=False):
    w = synth.Workload("t", batch=2, hq=4, hkv=2, head_dim=128, dtype="bf16", ctx=700,
                       budget=0, layers=1, seed=81, retention=True)
    d = synth.host_cache(w, n=700, cap=800)
    st = np.zeros((2, 2), np.int32) if start else None
    return d, st


def _run(d, st=None, t=None, ranges=None, nr=None):
    c = kvb.KVCache(to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_beta"]), to_dev(d["pos"]),
                    to_dev(d["len"]), start=None if st is None else to_dev(st))
    f = kvb.kv_check_cache(c, t=None if t is None else to_dev(t),
                           ranges=None if ranges is None else to_dev(ranges),
                           n_ranges=None if nr is None else to_dev(nr))
    torch.cuda.synchronize()
    return to_host(f)


def test_check_clean_cache():
    d, st = _base(start=True)
    rg = np.array([[[5, 9], [9, 30]], [[100, 200], [0, 0]]], np.int32)
    f = _run(d, st, t=np.array([700, 700], np.int32), ranges=rg, nr=np.array([2, 1], np.int32))
    assert not f.any(), f


def test_check_each_violation():
    cases = []
    d, _ = _base()
    d["len"][1, 0] = 801                                    # len above cap
    d["pos"][1, 0, 700:] = np.arange(700, 800)              # (clamped to cap: valid slots)
    cases.append(("len", d, None, {}, (1, 0)))
    d, st = _base(start=True)
    st[0, 1] = 800                                          # start outside [0, cap)
    cases.append(("start", d, st, {}, (0, 1)))
    d, _ = _base()
    d["pos"][0, 0, 300] = d["pos"][0, 0, 299]               # repeated position
    cases.append(("pos_order", d, None, {}, (0, 0)))
    d, _ = _base()
    d["pos"][1, 1, 10], d["pos"][1, 1, 11] = 11, 10         # swapped positions
    cases.append(("pos_order", d, None, {}, (1, 1)))
    d, _ = _base()
    cases.append(("pos_after_t", d, None, {"t": np.array([700, 600], np.int32)}, "b1"))
    d, _ = _base()
    d["log_beta"][0, 1, 5] = np.nan
    cases.append(("log_beta_nan", d, None, {}, (0, 1)))
    d, _ = _base()
    d["log_beta"][1, 0, 699] = 0.25
    cases.append(("log_beta_positive", d, None, {}, (1, 0)))
    d, _ = _base()
    d["log_beta"][1, 0, 750] = np.nan                        # beyond len: not live, no flag
    cases.append((None, d, None, {}, None))
    for bad_rg in ([[[9, 5]]], [[[1, 10], [5, 20]]], [[[1, 10], [0, 2]]]):
        d, _ = _base()
        rg = np.zeros((2, 2, 2), np.int32)
        rg[0, :len(bad_rg[0])] = np.array(bad_rg[0], np.int32)
        cases.append(("ranges", d, None, {"ranges": rg,
                                          "nr": np.array([len(bad_rg[0]), 0], np.int32)}, "b0"))
    d, _ = _base()
    cases.append(("ranges", d, None, {"ranges": np.zeros((2, 2, 2), np.int32),
                                      "nr": np.array([0, 3], np.int32)}, "b1"))
    for name, d, st, kw, where in cases:
        say("check case", name, where)
        f = _run(d, st, **kw)
        want = np.zeros((2, 2), np.int32)
        if name is not None:
            if where == "b0":
                want[0, :] = BITS[name]
            elif where == "b1":
                want[1, :] = BITS[name]
            else:
                want[where] = BITS[name]
        assert np.array_equal(f, want), (name, f, want)
