"""The C ABI: the library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

import bounded_decode_attention_amd as kvb
from bounded_decode_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvbound.h")

needs_lib = pytest.mark.skipif(not os.path.exists(kvb.library_path()),
                               reason="libkvbound.so not built")


def _has_gpu():
    import torch
    return torch.cuda.is_available()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("kv_attn_decode", "kv_evict_to_budget", "kv_erase_ranges", "asm_lookup_merge"):
        assert n in names


@needs_lib
def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(kvb.library_path())
    for name in declared_functions():
        assert hasattr(L, name), name


@needs_lib
def test_strerror():
    assert kvb.strerror(0) == "ok"
    for s in range(-7, 0):
        assert kvb.strerror(s) not in ("", "unknown status")
    assert kvb.strerror(-99) == "unknown status"


def _desc(**kw):
    d = dict(k=4096, v=8192, log_beta=None, pos=12288, len=16384, B=2, Hkv=2, cap=100, D=128,
             dtype=1)
    d.update(kw)
    return _lib._Cache(d["k"], d["v"], d["log_beta"], d["pos"], d["len"], d["B"], d["Hkv"],
                       d["cap"], d["D"], d["dtype"])


@needs_lib
def test_workspace_sizes_host_only():
    L = kvb.library()
    c = _desc()
    P = L.kv_attn_decode_splits(ctypes.byref(c), 8)
    assert P == 1  # 100-slot cache: a split covers at least 256 slots
    assert L.kv_attn_decode_splits(ctypes.byref(_desc(cap=2080, B=32, Hkv=8)), 32) == 8
    assert L.kv_attn_decode_splits(ctypes.byref(_desc(cap=32800, B=16, Hkv=8)), 32) == 16
    assert L.kv_attn_decode_workspace(ctypes.byref(c), 8, 0) >= 256 + 2 * 8 * P * 130 * 4
    assert L.kv_evict_workspace(ctypes.byref(c), 10) > 256
    assert L.kv_erase_workspace(ctypes.byref(c)) >= L.kv_evict_workspace(ctypes.byref(c), 10)
    assert L.asm_lookup_merge_workspace(32, 32, 8, 128, 4096) > 256
    assert L.kv_evict_workspace(ctypes.byref(c), -1) == 0
    assert L.asm_lookup_merge_workspace(1, 3, 2, 128, 16) == 0


def test_size_queries_reject_dimensions_the_calls_reject():
    """Size queries on descriptors the entry points would refuse return 0 instead of
    dividing by zero or overflowing (found by the sanitizer build of the host code)."""
    L = kvb.library()
    for bad in (_desc(Hkv=0), _desc(B=0), _desc(cap=0), _desc(cap=1 << 30),
                _desc(B=1 << 15, Hkv=1 << 15)):
        assert L.kv_attn_decode_splits(ctypes.byref(bad), 8) == 0
        assert L.kv_attn_decode_workspace(ctypes.byref(bad), 8, 0) == 0
        assert L.kv_attn_decode_asm_workspace(ctypes.byref(bad), 8, 0, 256) == 0
        assert L.kv_attn_decode_asm_splits(ctypes.byref(bad), 8, 256) == 0
        assert L.kv_evict_workspace(ctypes.byref(bad), 10) == 0
        assert L.kv_erase_workspace(ctypes.byref(bad)) == 0
        assert L.kv_latent_absorb_workspace(ctypes.byref(bad)) == 0
    c = _desc()
    assert L.kv_attn_decode_workspace(ctypes.byref(c), 8, -1) == 0
    # more query rows per KV head than the lookups take (B * G > 65536)
    assert L.kv_attn_decode_asm_workspace(ctypes.byref(_desc(B=1 << 17, Hkv=1)), 4, 0, 256) == 0
    assert L.asm_lookup_merge_workspace(1 << 30, 8, 2, 128, 256) == 0
    assert L.asm_lookup_merge_workspace(1, 8, 2, 128, 1 << 24) == 0
    assert L.asm_lookup_merge_hier_workspace(1 << 30, 8, 2, 16, 4) == 0
    # one chunk per token at most, whatever the chunk count asked for
    assert L.asm_prefix_states_workspace(2, 1024, 128, 512, 2 ** 31 - 1) == \
        L.asm_prefix_states_workspace(2, 1024, 128, 512, 512)


@needs_lib
def test_invalid_arguments_rejected_before_launch():
    """Fake (never dereferenced) pointers: validation fails first, nothing runs."""
    L = kvb.library()
    P = ctypes.c_void_p
    ws = P(4096)
    good = _desc()
    # kv_attn_decode
    args = [P(64), 8, P(72), 0.0, None, None, None, 0, P(80), P(88), ws, 1 << 30, None]
    assert L.kv_attn_decode(None, *args) == -1
    assert L.kv_attn_decode(ctypes.byref(good), P(64), 7, *args[2:]) == -1      # Hq % Hkv
    assert L.kv_attn_decode(ctypes.byref(_desc(D=96)), *args) == -2            # bf16 D=96
    assert L.kv_attn_decode(ctypes.byref(_desc(dtype=5)), *args) == -2
    assert L.kv_attn_decode(ctypes.byref(_desc(cap=0)), *args) == -1
    assert L.kv_attn_decode(ctypes.byref(_desc(pos=None)), *args) == -1
    a2 = list(args)
    a2[4] = P(8)                                                              # k_new w/o v_new
    assert L.kv_attn_decode(ctypes.byref(good), *a2) == -1
    a3 = list(args)
    a3[7] = 5000                                                              # num_splits
    assert L.kv_attn_decode(ctypes.byref(good), *a3) == -1
    a4 = list(args)
    a4[11] = 16                                                               # ws too small
    assert L.kv_attn_decode(ctypes.byref(good), *a4) == -4
    # kv_evict_to_budget
    assert L.kv_evict_to_budget(ctypes.byref(good), P(8), -1, None, 0, None, ws, 1 << 30, None) == -1
    assert L.kv_evict_to_budget(ctypes.byref(good), None, 5, None, 0, None, ws, 1 << 30, None) == -1
    assert L.kv_evict_to_budget(ctypes.byref(good), P(8), 5, None, 0, None, ws, 8, None) == -4
    # kv_erase_ranges
    assert L.kv_erase_ranges(ctypes.byref(good), None, P(8), 3, None, ws, 1 << 30, None) == -1
    assert L.kv_erase_ranges(ctypes.byref(good), P(8), None, 3, None, ws, 1 << 30, None) == -1
    # asm_lookup_merge
    base = [P(8), 2, 8, 2, 128, P(8), P(8), P(8), 64, P(8), P(8), P(8), P(8), None, ws, 1 << 30, None]
    bad = list(base)
    bad[4] = 96
    assert L.asm_lookup_merge(*bad) == -2
    bad = list(base)
    bad[2] = 7
    assert L.asm_lookup_merge(*bad) == -1
    bad = list(base)
    bad[0] = None
    assert L.asm_lookup_merge(*bad) == -1


@needs_lib
def test_hier_lookup_arguments_rejected_before_launch():
    """Fake pointers: the two-level lookup's validation runs on the host first."""
    L = kvb.library()
    P = ctypes.c_void_p
    ws = P(4096)
    # q, B, Hq, Hkv, D, c1, K1, offs, centroids, kid, K, m, abar, log_zbar, self_out,
    # self_lse, out, out_lse, idx, ws, ws_bytes, stream
    base = [P(8), 2, 8, 2, 128, P(8), 64, P(8), P(8), P(8), 4096, 16, P(8), P(8), P(8), P(8),
            P(8), P(8), None, ws, 1 << 30, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.asm_lookup_merge_hier(*a)

    assert call(a4=96) == -2                 # D
    assert call(a2=7) == -1                  # Hq % Hkv
    assert call(a6=0) == -1                  # K1
    assert call(a6=513) == -1                # K1 above 512
    assert call(a11=0) == -1                 # m
    assert call(a11=65) == -1                # m above K1
    assert call(a7=None) == -1               # offs
    assert call(a9=None) == -1               # kid
    assert call(a10=1 << 24) == -1           # K
    assert call(a20=64) == -4                # workspace too small
    assert L.asm_lookup_merge_hier_workspace(2, 8, 2, 64, 16) > 256
    assert L.asm_lookup_merge_hier_workspace(2, 8, 2, 64, 65) == 0
    assert L.asm_lookup_merge_hier_workspace(2, 8, 2, 600, 16) == 0


@needs_lib
def test_build_entry_points_reject_arguments_before_launch():
    """Fake pointers: the memory-build calls validate on the host first."""
    L = kvb.library()
    P = ctypes.c_void_p
    ws = P(4096)
    # asm_prefix_states: q, H, N, D, k, v, L, chunks, scale, a, lse, ws, ws_bytes, stream
    pre = [P(8), 2, 100, 128, P(8), P(8), 300, 4, 0.0, P(8), P(8), ws, 1 << 30, None]

    def call(fn, base, **kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return fn(*a)

    f = L.asm_prefix_states
    assert call(f, pre, a3=96) == -2          # D
    assert call(f, pre, a1=0) == -1           # H
    assert call(f, pre, a2=1 << 24) == -1     # N
    assert call(f, pre, a7=0) == -1           # chunks
    assert call(f, pre, a6=-1) == -1          # L
    assert call(f, pre, a4=None) == -1        # k with L > 0
    assert call(f, pre, a9=None) == -1        # a
    assert call(f, pre, a12=64) == -4         # workspace too small for 4 chunk states
    # one chunk: V^T of the 300 tokens (padded to 320 keys), the per-tile (5 tiles of
    # 64 keys) and per-chunk range words of every dimension
    assert L.asm_prefix_states_workspace(2, 100, 128, 300, 1) == (256 + 2 * 128 * 320 * 2 +
                                                                2 * 5 * 128 * 4 + 2 * 128 * 4)
    assert L.asm_prefix_states_workspace(2, 100, 128, 0, 4) == 256
    # 300 tokens in 4 chunks of 75 (V^T padded to 128 keys each): 4 states per query
    assert L.asm_prefix_states_workspace(2, 100, 128, 300, 4) >= (256 + 2 * 4 * 128 * 128 * 2 +
                                                                4 * 200 * 129 * 4)
    # asm_kmeans: x, H, N, D, centroids, K, iters, assign, counts, cent_bf16, ws, ws_bytes, stream
    km = [P(8), 2, 100, 128, P(8), 16, 3, P(8), None, None, ws, 1 << 30, None]
    f = L.asm_kmeans
    assert call(f, km, a3=64 + 8) == -2       # D
    assert call(f, km, a5=0) == -1            # K
    assert call(f, km, a6=0) == -1            # iters
    assert call(f, km, a7=None) == -1         # assign
    assert call(f, km, a4=None) == -1         # centroids
    assert call(f, km, a11=100) == -4         # workspace
    assert L.asm_kmeans_workspace(2, 16, 128) >= 256 + 2 * 2 * 16 * 128 * 2
    # asm_aggregate_states: assign, a, lse, H, N, D, K, abar, log_zbar, stream
    ag = [P(8), P(8), P(8), 2, 100, 128, 16, P(8), P(8), None]
    f = L.asm_aggregate_states
    assert call(f, ag, a5=32) == -2
    assert call(f, ag, a6=0) == -1
    assert call(f, ag, a0=None) == -1
    assert call(f, ag, a8=None) == -1
    # asm_build_memory: q, H, N, D, k, v, L, chunks, scale, centroids, K, iters,
    # centroids_bf16, abar, log_zbar, assign, ws, ws_bytes, stream
    bm = [P(8), 2, 100, 128, P(8), P(8), 300, 4, 0.0, P(8), 16, 3, P(8), P(8), P(8), P(8), ws,
          1 << 30, None]
    f = L.asm_build_memory
    assert call(f, bm, a3=96) == -2
    assert call(f, bm, a11=0) == -1
    assert call(f, bm, a12=None) == -1
    assert call(f, bm, a17=1024) == -4
    assert (L.asm_build_memory_workspace(2, 100, 128, 300, 4, 16) >=
            L.asm_prefix_states_workspace(2, 100, 128, 300, 4) + L.asm_kmeans_workspace(2, 16, 128))


@needs_lib
def test_latent_entry_points_reject_arguments_before_launch():
    L = kvb.library()
    P = ctypes.c_void_p
    c = _desc()
    ws = P(4096)
    wsz = L.kv_latent_absorb_workspace(ctypes.byref(c))
    assert wsz > 256
    ev = L.kv_evict_workspace(ctypes.byref(c), 50)
    # cache, M, ws_evict, ws_evict_bytes, lam, mem_M, mem_b, ws, ws_bytes, stream
    base = [ctypes.byref(c), 50, P(8), ev, 0.99, P(8), P(8), ws, wsz, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.kv_latent_absorb(*a)

    assert call(a4=0.0) == -1                 # lam outside (0, 1]
    assert call(a4=1.5) == -1
    assert call(a5=None) == -1                # mem_M
    assert call(a2=None) == -1                # plan workspace
    assert call(a3=ev - 1) == -4              # plan workspace too small
    assert call(a8=wsz - 1) == -4             # own workspace too small
    c32 = _desc(dtype=0)
    assert L.kv_latent_absorb(ctypes.byref(c32), 50, P(8), 1 << 40, 0.99, P(8), P(8), ws,
                              1 << 40, None) == -2
    # q, B, Hq, Hkv, D, mem_M, mem_b, W_o, w_g, c_g, eps, out, stream
    rd = [P(8), 2, 8, 2, 128, P(8), P(8), P(8), P(8), P(8), 1e-6, P(8), None]
    a = list(rd)
    a[4] = 96
    assert L.kv_latent_read(*a) == -2
    a = list(rd)
    a[2] = 7
    assert L.kv_latent_read(*a) == -1
    a = list(rd)
    a[10] = -1.0
    assert L.kv_latent_read(*a) == -1
    a = list(rd)
    a[7] = None
    assert L.kv_latent_read(*a) == -1


def test_cache_descriptor_layout_matches_header(tmp_path):
    """The ctypes descriptor has the C struct's size and field offsets (compiled from
    the header with the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f[0] for f in _lib._Cache._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kvbound.h"\nint main(void) {\n'
                   '  printf("size %zu\\n", sizeof(kvb_cache));\n'
                   + "".join(f'  printf("{f} %zu\\n", offsetof(kvb_cache, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(_lib._Cache)
    for f in fields:
        assert int(out[f]) == getattr(_lib._Cache, f).offset, f


@needs_lib
def test_fused_asm_entry_rejects_arguments_before_launch():
    """kv_attn_decode_asm: fake (never dereferenced) pointers; validation first."""
    L = kvb.library()
    P = ctypes.c_void_p
    good = _desc()
    need = L.kv_attn_decode_asm_workspace(ctypes.byref(good), 8, 0, 4096)
    assert need > L.kv_attn_decode_workspace(ctypes.byref(good), 8, 0)
    args = lambda **kw: [kw.get("q", P(64)), 8, P(72), 0.0, None, None, None, 0,  # noqa: E731
                         kw.get("cent", P(8)), P(16), P(24), kw.get("K", 4096), P(80), P(88),
                         None, P(4096), kw.get("ws_bytes", need), None]
    assert L.kv_attn_decode_asm(ctypes.byref(good), *args(cent=None)) == -1
    assert L.kv_attn_decode_asm(ctypes.byref(good), *args(q=None)) == -1
    assert L.kv_attn_decode_asm(ctypes.byref(good), *args(K=0)) == -1
    assert L.kv_attn_decode_asm(ctypes.byref(_desc(dtype=0, D=64)), *args()) == -2  # f32 cache
    assert L.kv_attn_decode_asm(ctypes.byref(good), *args(ws_bytes=need - 1)) == -4
    assert L.kv_attn_decode_asm_workspace(ctypes.byref(good), 7, 0, 4096) == 0    # Hq % Hkv
    # default splits: what one round of 2048 waves leaves beside the scan's tasks
    asm_c = _desc(B=32, Hkv=8, cap=2080)
    assert L.kv_attn_decode_splits(ctypes.byref(asm_c), 32) == 8
    assert L.kv_attn_decode_asm_splits(ctypes.byref(asm_c), 32, 4096) == 4
    assert L.kv_attn_decode_asm_splits(ctypes.byref(asm_c), 31, 4096) == 0
    assert L.kv_attn_decode_asm_splits(ctypes.byref(_desc(B=32, Hkv=8, cap=2080, D=64)), 32,
                                       4096) == 8


@needs_lib
def test_noalloc_entry_rejects_arguments_before_launch():
    """kv_attn_decode_noalloc: fake pointers; invalid arguments, and a call that
    would need more than the fixed device scratch, are refused on the host."""
    L = kvb.library()
    P = ctypes.c_void_p
    good = _desc()
    # q, Hq, t, scale, k_new, v_new, log_beta_new, num_splits, out, lse, status, stream
    args = [P(64), 8, P(72), 0.0, None, None, None, 0, P(80), P(88), None, None]
    assert L.kv_attn_decode_noalloc(None, *args) == -1
    assert L.kv_attn_decode_noalloc(ctypes.byref(good), P(64), 7, *args[2:]) == -1
    a = list(args)
    a[7] = 5000
    assert L.kv_attn_decode_noalloc(ctypes.byref(good), *a) == -1
    a = list(args)
    a[8] = None
    assert L.kv_attn_decode_noalloc(ctypes.byref(good), *a) == -1
    big = _desc(B=64, Hkv=8, cap=8192)
    assert L.kv_attn_decode_workspace(ctypes.byref(big), 64, 32) > kvb.NOALLOC_SCRATCH_BYTES
    a = [P(64), 64, P(72), 0.0, None, None, None, 32, P(80), P(88), None, None]
    assert L.kv_attn_decode_noalloc(ctypes.byref(big), *a) == -4


def test_noalloc_limit_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define\s+KVB_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == kvb.NOALLOC_SCRATCH_BYTES


@needs_lib
@pytest.mark.skipif(_has_gpu(), reason="a GPU is present")
def test_valid_calls_without_a_gpu_return_edevice():
    """Arguments that pass every host check reach the device check: without a HIP
    device the call returns KVB_EDEVICE (-5) and launches nothing."""
    L = kvb.library()
    P = ctypes.c_void_p
    good = _desc()
    ws = P(4096)
    args = [P(64), 8, P(72), 0.0, None, None, None, 0, P(80), P(88), ws, 1 << 30, None]
    assert L.kv_attn_decode(ctypes.byref(good), *args) == -5
    assert L.kv_attn_decode_noalloc(ctypes.byref(good), P(64), 8, P(72), 0.0, None, None, None,
                                    0, P(80), P(88), None, None) == -5
    assert L.kv_evict_to_budget(ctypes.byref(good), P(8), 5, None, 0, None, ws, 1 << 30,
                                None) == -5
    assert L.kv_append(ctypes.byref(good), P(8), P(8), None, P(8), ws, 256, None) == -5


@needs_lib
def test_check_cache_rejects_arguments_before_launch():
    L = kvb.library()
    P = ctypes.c_void_p
    good = _desc()
    assert L.kv_check_cache(None, None, None, None, 0, P(8), None) == -1
    assert L.kv_check_cache(ctypes.byref(good), None, None, None, 0, None, None) == -1  # flags
    assert L.kv_check_cache(ctypes.byref(good), None, None, None, -1, P(8), None) == -1
    assert L.kv_check_cache(ctypes.byref(good), None, None, P(8), 3, P(8), None) == -1  # ranges
    assert L.kv_check_cache(ctypes.byref(_desc(pos=None)), None, None, None, 0, P(8), None) == -1


@needs_lib
def test_plan_one_entries_reject_arguments_before_launch():
    """kv_attn_decode_plan_one / kv_evict_one_apply: fake pointers; a missing or
    short eviction workspace, bad splits or budget are refused on the host, and
    valid arguments without a GPU stop at the device check."""
    L = kvb.library()
    P = ctypes.c_void_p
    good = _desc()
    need = L.kv_evict_one_workspace(ctypes.byref(good), 0)
    assert need > 256
    assert L.kv_evict_one_workspace(ctypes.byref(good), 7) > need - 1
    assert L.kv_evict_one_workspace(ctypes.byref(good), -1) == 0
    assert L.kv_evict_one_workspace(None, 0) == 0
    wsa = L.kv_attn_decode_workspace(ctypes.byref(good), 8, 0)

    def plan(ws_e=P(8192), ws_e_bytes=need, splits=0, c=good):
        return L.kv_attn_decode_plan_one(ctypes.byref(c), P(64), 8, P(72), 0.0, None, None,
                                         None, splits, P(80), P(88), P(4096), wsa, ws_e,
                                         ws_e_bytes, None)
    assert plan(ws_e=None) == -4
    assert plan(ws_e_bytes=need - 1) == -4
    assert plan(splits=5000) == -1
    assert plan(c=_desc(B=300, Hkv=256)) == -2     # B * Hkv above 65535

    def apply(t=P(72), M=5, ws=P(8192), ws_bytes=need, me=0):
        return L.kv_evict_one_apply(ctypes.byref(good), t, M, None, me, None, ws, ws_bytes,
                                    None)
    assert apply(t=None) == -1
    assert apply(M=-1) == -1
    assert apply(me=-1) == -1
    assert apply(ws=None) == -4
    assert apply(ws_bytes=300) == -4
    need1 = L.kv_attn_decode_evict_one_workspace(ctypes.byref(good), 8, 0)
    assert need1 > wsa
    assert L.kv_attn_decode_evict_one_workspace(ctypes.byref(good), 7, 0) == 0   # Hq % Hkv

    def one(M=5, splits=0, ws=P(4096), ws_bytes=need1, me=0, c=good):
        # q, Hq, t, scale, k_new, v_new, log_beta_new, M, num_splits, out, lse,
        # evicted_pos, max_evict, n_evicted, ws, ws_bytes, stream
        return L.kv_attn_decode_evict_one(ctypes.byref(c), P(64), 8, P(72), 0.0, None, None,
                                          None, M, splits, P(80), P(88), None, me, None, ws,
                                          ws_bytes, None)
    assert one(M=-1) == -1
    assert one(me=-2) == -1
    assert one(splits=4097) == -1
    assert one(ws=None) == -4
    assert one(ws_bytes=need1 - 1) == -4
    assert one(c=_desc(B=300, Hkv=256)) == -2
    if not _has_gpu():
        assert plan() == -5
        assert apply() == -5
        assert one() == -5


@needs_lib
def test_paged_entries_reject_arguments_before_launch():
    """kv_attn_decode_paged / kv_erase_ranges_paged: fake pointers; missing page
    arrays, a start array, a capacity off the 32-slot pages, unsupported shapes and
    short workspaces are refused on the host; valid calls without a GPU stop at the
    device check.  The erase workspace formula."""
    L = kvb.library()
    P = ctypes.c_void_p
    good = _desc(cap=128)
    pages = _lib._Pages(200, 208, 216, 6)
    no_fill = _lib._Pages(200, None, 216, 6)
    wsa = L.kv_attn_decode_workspace(ctypes.byref(good), 8, 0)

    def attn(c=good, pg=pages, Hq=8, splits=0, ws_bytes=wsa):
        # q, Hq, t, scale, k_new, v_new, log_beta_new, spare, num_splits, out, lse, ws
        return L.kv_attn_decode_paged(ctypes.byref(c), None if pg is None else ctypes.byref(pg),
                                      P(64), Hq, P(72), 0.0, None, None, None, None, splits,
                                      P(80), P(88), P(4096), ws_bytes, None)
    assert attn(pg=None) == -1
    assert attn(pg=no_fill) == -1
    assert attn(pg=_lib._Pages(200, 208, 216, 0)) == -1
    assert attn(c=_desc(cap=100)) == -1                 # not whole pages
    st = _desc(cap=128)
    st.start = 32
    assert attn(c=st) == -1
    assert attn(Hq=7) == -1
    assert attn(Hq=32) == -2                            # group of 16
    assert attn(c=_desc(cap=128, D=64)) == -2
    assert attn(splits=4097) == -1
    assert attn(ws_bytes=300) == -4
    need = L.kv_erase_paged_workspace(ctypes.byref(good), ctypes.byref(pages))
    U, mp, NB = 4, 6, 1
    a256 = lambda x: (x + 255) // 256 * 256
    assert need == 256 + 3 * a256(U * mp * 4) + a256(U * NB * 12)
    big = _lib._Pages(200, 208, 216, 1000)
    assert L.kv_erase_paged_workspace(ctypes.byref(good), ctypes.byref(big)) == \
        256 + 3 * a256(U * 1000 * 4) + a256(U * 4 * 12)
    assert L.kv_erase_paged_workspace(ctypes.byref(good), None) == 0

    def erase(c=good, pg=pages, R=2, ranges=P(300), nr=P(308), ws=P(4096), ws_bytes=need):
        return L.kv_erase_ranges_paged(ctypes.byref(c), None if pg is None else ctypes.byref(pg),
                                       ranges, nr, R, None, ws, ws_bytes, None)
    assert erase(pg=None) == -1
    assert erase(pg=no_fill) == -1
    assert erase(c=_desc(cap=100)) == -1
    assert erase(c=st) == -1
    assert erase(R=-1) == -1
    assert erase(ranges=None) == -1
    assert erase(nr=None) == -1
    assert erase(ws=None) == -4
    assert erase(ws_bytes=need - 1) == -4
    assert erase(c=_desc(cap=128, B=300, Hkv=256)) == -2   # B * Hkv above 65535
    if not _has_gpu():
        assert attn() == -5
        assert erase() == -5
        assert erase(R=0, ranges=None) == -5


@needs_lib
def test_misaligned_pointers_rejected():
    """Cache arrays and the query are read 16 bytes at a time: a pointer off a
    16-byte boundary is refused on the host (KVB_EINVAL) before any launch."""
    L = kvb.library()
    P = ctypes.c_void_p
    ws = P(1 << 20)
    args = [P(64), 8, P(72), 0.0, None, None, None, 0, P(80), P(88), ws, 1 << 30, None]
    for kw in (dict(k=4100), dict(v=8196), dict(pos=12292), dict(log_beta=20488)):
        assert L.kv_attn_decode(ctypes.byref(_desc(**kw)), *args) == -1, kw
        assert L.kv_evict_to_budget(ctypes.byref(_desc(**kw)), P(8), 5, None, 0, None, ws,
                                    1 << 30, None) == -1, kw
    assert L.kv_attn_decode(ctypes.byref(_desc()), P(68), *args[1:]) == -1
    if not _has_gpu():
        assert L.kv_attn_decode(ctypes.byref(_desc(log_beta=20480)), *args) == -5


@needs_lib
def test_check_pages_rejects_arguments_before_launch():
    L = kvb.library()
    P = ctypes.c_void_p
    good = _desc(cap=128)
    pages = _lib._Pages(200, 208, 216, 6)

    def chk(c=good, pg=pages, flags=P(512)):
        return L.kv_check_pages(ctypes.byref(c), None if pg is None else ctypes.byref(pg),
                                None, flags, None)
    assert chk(flags=None) == -1
    assert chk(pg=None) == -1
    assert chk(pg=_lib._Pages(200, None, 216, 6)) == -1
    assert chk(pg=_lib._Pages(200, 208, 216, 0)) == -1
    assert chk(pg=_lib._Pages(200, 208, 216, (1 << 25) + 1)) == -1
    assert chk(c=_desc(cap=100)) == -1
    st = _desc(cap=128)
    st.start = 32
    assert chk(c=st) == -1
    if not _has_gpu():
        assert chk() == -5
