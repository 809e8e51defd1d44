"""ctypes marshalling for libkvbound.so (see include/kvbound.h for the contract)."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvbound.so")
_lib = None

KVB_F32, KVB_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20    # KVB_NOALLOC_SCRATCH_BYTES in kvbound.h


class KVBError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("log_beta", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("len", ctypes.c_void_p), ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("cap", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("start", ctypes.c_void_p)]


class _Pages(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("fill", ctypes.c_void_p),
                ("n_pages", ctypes.c_void_p), ("max_pages", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def library():
    """The loaded shared library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libkvbound.so is not built ({_LIB_PATH}); run "
                              "python -m bounded_decode_attention_amd.build")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        CP = ctypes.POINTER(_Cache)
        PP = ctypes.POINTER(_Pages)
        sigs = {
            "kvb_strerror": (ctypes.c_char_p, [I32]),
            "kv_attn_decode_splits": (I32, [CP, I32]),
            "kv_attn_decode_workspace": (SZ, [CP, I32, I32]),
            "kv_evict_workspace": (SZ, [CP, I32]),
            "kv_erase_workspace": (SZ, [CP]),
            "asm_lookup_merge_workspace": (SZ, [I32, I32, I32, I32, I32]),
            "asm_lookup_merge_hier_workspace": (SZ, [I32, I32, I32, I32, I32]),
            "kv_attn_decode": (I32, [CP, P, I32, P, F, P, P, P, I32, P, P, P, SZ, P]),
            "kv_attn_decode_noalloc": (I32, [CP, P, I32, P, F, P, P, P, I32, P, P, P, P]),
            "kv_check_cache": (I32, [CP, P, P, P, I32, P, P]),
            "kv_check_pages": (I32, [CP, PP, P, P, P]),
            "kv_attn_decode_asm_workspace": (SZ, [CP, I32, I32, I32]),
            "kv_attn_decode_asm_splits": (I32, [CP, I32, I32]),
            "kv_attn_decode_asm": (I32, [CP, P, I32, P, F, P, P, P, I32, P, P, P, I32, P, P, P,
                                         P, SZ, P]),
            "kv_evict_to_budget": (I32, [CP, P, I32, P, I32, P, P, SZ, P]),
            "kv_evict_plan": (I32, [CP, P, I32, P, I32, P, P, SZ, P]),
            "kv_evict_apply": (I32, [CP, I32, P, SZ, P]),
            "kv_evict_one": (I32, [CP, P, I32, P, I32, P, P]),
            "kv_evict_one_workspace": (SZ, [CP, I32]),
            "kv_attn_decode_plan_one": (I32, [CP, P, I32, P, F, P, P, P, I32, P, P, P, SZ, P,
                                              SZ, P]),
            "kv_evict_one_apply": (I32, [CP, P, I32, P, I32, P, P, SZ, P]),
            "kv_attn_decode_evict_one_workspace": (SZ, [CP, I32, I32]),
            "kv_attn_decode_evict_one": (I32, [CP, P, I32, P, F, P, P, P, I32, I32, P, P, P, I32,
                                               P, P, SZ, P]),
            "kv_append": (I32, [CP, P, P, P, P, P, SZ, P]),
            "kv_attn_decode_compact": (I32, [CP, P, I32, P, F, I32, I32, I32, P, P, P, SZ, P, SZ,
                                             P]),
            "kv_erase_ranges": (I32, [CP, P, P, I32, P, P, SZ, P]),
            "kv_attn_decode_paged": (I32, [CP, PP, P, I32, P, F, P, P, P, P, I32, P, P, P, SZ,
                                           P]),
            "kv_erase_paged_workspace": (SZ, [CP, PP]),
            "kv_erase_ranges_paged": (I32, [CP, PP, P, P, I32, P, P, SZ, P]),
            "asm_lookup_merge": (I32, [P, I32, I32, I32, I32, P, P, P, I32, P, P, P, P, P, P,
                                       SZ, P]),
            "asm_lookup_merge_hier": (I32, [P, I32, I32, I32, I32, P, I32, P, P, P, I32, I32, P,
                                            P, P, P, P, P, P, P, SZ, P]),
            "asm_prefix_states_workspace": (SZ, [I32, I32, I32, I32, I32]),
            "asm_kmeans_workspace": (SZ, [I32, I32, I32]),
            "asm_build_memory_workspace": (SZ, [I32, I32, I32, I32, I32, I32]),
            "asm_prefix_states": (I32, [P, I32, I32, I32, P, P, I32, I32, F, P, P, P, SZ, P]),
            "asm_kmeans": (I32, [P, I32, I32, I32, P, I32, I32, P, P, P, P, SZ, P]),
            "asm_aggregate_states": (I32, [P, P, P, I32, I32, I32, I32, P, P, P]),
            "asm_build_memory": (I32, [P, I32, I32, I32, P, P, I32, I32, F, P, I32, I32, P, P, P,
                                       P, P, SZ, P]),
            "kv_latent_absorb_workspace": (SZ, [CP]),
            "kv_latent_absorb": (I32, [CP, I32, P, SZ, F, P, P, P, SZ, P]),
            "kv_latent_read": (I32, [P, I32, I32, I32, I32, P, P, P, P, P, F, P, P]),
            "kvb_trace_enable": (I32, [I32, I32]),
            "kvb_trace_read": (I32, [P, P, I32]),
            "kvb_trace_reset": (None, []),
            "kvb_trace_disable": (None, []),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return library().kvb_strerror(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != 0:
        raise KVBError(status, where)


def _need(t, name, dtype=None, device=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


class KVCache:
    """One layer's cache tensors (all on the same device, contiguous).

    k, v      [B][Hkv][cap][D] bfloat16 or float32
    log_beta  [B][Hkv][cap] float32, or None (beta == 1)
    pos       [B][Hkv][cap] int32
    length    [B][Hkv] int32 (device)
    start     [B][Hkv] int32 (device) first live slot per head, or None (all 0);
              eviction then compacts each head toward whichever end moves fewer
              rows and updates start
    """

    def __init__(self, k, v, log_beta, pos, length, start=None):
        _need(k, "k")
        _need(v, "v", k.dtype)
        if k.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("k/v dtype must be bfloat16 or float32")
        if k.shape != v.shape or k.dim() != 4:
            raise ValueError("k, v must both be [B][Hkv][cap][D]")
        B, H, cap, D = k.shape
        if log_beta is not None:
            _need(log_beta, "log_beta", torch.float32)
            if tuple(log_beta.shape) != (B, H, cap):
                raise ValueError("log_beta must be [B][Hkv][cap]")
        _need(pos, "pos", torch.int32)
        _need(length, "length", torch.int32)
        if tuple(pos.shape) != (B, H, cap) or tuple(length.shape) != (B, H):
            raise ValueError("pos must be [B][Hkv][cap], length [B][Hkv]")
        if start is not None:
            _need(start, "start", torch.int32)
            if tuple(start.shape) != (B, H):
                raise ValueError("start must be [B][Hkv]")
        self.k, self.v, self.log_beta, self.pos, self.length = k, v, log_beta, pos, length
        self.start = start
        self.B, self.Hkv, self.cap, self.D = B, H, cap, D
        self.dtype = KVB_BF16 if k.dtype == torch.bfloat16 else KVB_F32
        self._desc = _Cache(k.data_ptr(), v.data_ptr(),
                            None if log_beta is None else log_beta.data_ptr(),
                            pos.data_ptr(), length.data_ptr(), B, H, cap, D, self.dtype,
                            None if start is None else start.data_ptr())

    @classmethod
    def from_dict(cls, d):
        return cls(d["k"], d["v"], d.get("log_beta"), d["pos"], d["len"], d.get("start"))

    @property
    def desc(self):
        return ctypes.byref(self._desc)


class KVPages:
    """Page table of a paged cache (32-slot pages; see kvb_pages in kvbound.h).

    table    [B][Hkv][max_pages] int32 physical page of each logical page
    fill     [B][Hkv][max_pages] int32 live slots of each logical page (1..32)
    n_pages  [B][Hkv] int32 logical pages in use
    """

    def __init__(self, table, fill, n_pages):
        _need(table, "table", torch.int32)
        _need(fill, "fill", torch.int32)
        _need(n_pages, "n_pages", torch.int32)
        if table.dim() != 3 or fill.shape != table.shape or \
                tuple(n_pages.shape) != tuple(table.shape[:2]):
            raise ValueError("table, fill must be [B][Hkv][max_pages] and n_pages [B][Hkv]")
        self.table, self.fill, self.n_pages = table, fill, n_pages
        self.max_pages = table.shape[2]
        self._desc = _Pages(table.data_ptr(), fill.data_ptr(), n_pages.data_ptr(),
                            self.max_pages)

    @property
    def desc(self):
        return ctypes.byref(self._desc)


def _ws(ws, nbytes, device):
    """The caller's workspace (uint8 device tensor), or a new one of the needed size.
    A caller workspace that is too small is passed through; the library rejects it."""
    if ws is None:
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    return ws


def kv_attn_decode_splits(cache: KVCache, Hq: int) -> int:
    return int(library().kv_attn_decode_splits(cache.desc, Hq))


def kv_attn_decode_workspace(cache: KVCache, Hq: int, num_splits: int = 0) -> int:
    return int(library().kv_attn_decode_workspace(cache.desc, Hq, num_splits))


def kv_evict_workspace(cache: KVCache, M: int) -> int:
    return int(library().kv_evict_workspace(cache.desc, M))


def kv_erase_workspace(cache: KVCache) -> int:
    return int(library().kv_erase_workspace(cache.desc))


def asm_lookup_merge_workspace(B, Hq, Hkv, D, K) -> int:
    return int(library().asm_lookup_merge_workspace(B, Hq, Hkv, D, K))


def workspace_status(ws, stream=None) -> int:
    """The status word (int32 at byte 0) a call left in its workspace; waits for
    the stream first."""
    (stream or torch.cuda.current_stream()).synchronize()
    return int(ws[:4].view(torch.int32).item())


def _check_ws(ws, stream, where):
    _check(workspace_status(ws, stream), where)


def kv_attn_decode(cache: KVCache, q, t, scale: float = 0.0, k_new=None, v_new=None,
                   log_beta_new=None, num_splits: int = 0, out=None, lse=None, ws=None,
                   stream=None, check_status: bool = False):
    """Append (optional) + retention-biased GQA decode attention.  Returns (out, lse).
    check_status: wait for the call and raise if its status word reports a full head."""
    _need(q, "q", cache.k.dtype)
    _need(t, "t", torch.int32)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x is not None:
            _need(x, name, cache.k.dtype)
    if log_beta_new is not None:
        _need(log_beta_new, "log_beta_new", torch.float32)
    ws = _ws(ws, kv_attn_decode_workspace(cache, Hq, num_splits), q.device)
    st = library().kv_attn_decode(cache.desc, _ptr(q), Hq, _ptr(t), float(scale), _ptr(k_new),
                                  _ptr(v_new), _ptr(log_beta_new), int(num_splits), _ptr(out),
                                  _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_attn_decode")
    if check_status:
        _check_ws(ws, stream, "kv_attn_decode (device status)")
    return out, lse


def kv_attn_decode_noalloc(cache: KVCache, q, t, out, lse, scale: float = 0.0, k_new=None,
                           v_new=None, log_beta_new=None, num_splits: int = 0, status=None,
                           stream=None):
    """kv_attn_decode on the library's device-resident scratch (no workspace, nothing
    allocated here or in the library): out [B][Hq][D] f32 and lse [B][Hq] f32 are the
    caller's; status: optional int32 device tensor of one element that receives the
    call's status word."""
    _need(q, "q", cache.k.dtype)
    _need(t, "t", torch.int32)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out must be [B][Hq][D] and lse [B][Hq]")
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x is not None:
            _need(x, name, cache.k.dtype)
    if log_beta_new is not None:
        _need(log_beta_new, "log_beta_new", torch.float32)
    if status is not None:
        _need(status, "status", torch.int32)
    st = library().kv_attn_decode_noalloc(cache.desc, _ptr(q), Hq, _ptr(t), float(scale),
                                          _ptr(k_new), _ptr(v_new), _ptr(log_beta_new),
                                          int(num_splits), _ptr(out), _ptr(lse), _ptr(status),
                                          _stream(stream))
    if st == -4:
        raise KVBError(st, "kv_attn_decode_noalloc: the call needs more than the "
                       f"{NOALLOC_SCRATCH_BYTES >> 20} MiB device scratch")
    _check(st, "kv_attn_decode_noalloc")
    return out, lse


def kv_attn_decode_asm_splits(cache: KVCache, Hq: int, K: int) -> int:
    return int(library().kv_attn_decode_asm_splits(cache.desc, int(Hq), int(K)))


def kv_attn_decode_asm_workspace(cache: KVCache, Hq: int, num_splits: int, K: int) -> int:
    return int(library().kv_attn_decode_asm_workspace(cache.desc, Hq, num_splits, K))


def kv_attn_decode_asm(cache: KVCache, q, t, centroids, abar, log_zbar, scale: float = 0.0,
                       k_new=None, v_new=None, log_beta_new=None, num_splits: int = 0, out=None,
                       lse=None, idx=None, ws=None, stream=None):
    """kv_attn_decode then asm_lookup_merge on its state, the lookup's merge done by
    the attention's merge (see kv_attn_decode_asm in kvbound.h).  centroids, abar
    [Hkv][K][D] bf16; log_zbar [Hkv][K] f32.  Returns (out, lse, idx)."""
    _need(q, "q", torch.bfloat16)
    _need(t, "t", torch.int32)
    _need(centroids, "centroids", torch.bfloat16)
    _need(abar, "abar", torch.bfloat16)
    _need(log_zbar, "log_zbar", torch.float32)
    B, Hq, D = q.shape
    K = centroids.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _need(idx, "idx", torch.int32)
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x is not None:
            _need(x, name, torch.bfloat16)
    if log_beta_new is not None:
        _need(log_beta_new, "log_beta_new", torch.float32)
    ws = _ws(ws, kv_attn_decode_asm_workspace(cache, Hq, num_splits, K), q.device)
    st = library().kv_attn_decode_asm(cache.desc, _ptr(q), Hq, _ptr(t), float(scale),
                                      _ptr(k_new), _ptr(v_new), _ptr(log_beta_new),
                                      int(num_splits), _ptr(centroids), _ptr(abar),
                                      _ptr(log_zbar), int(K), _ptr(out), _ptr(lse), _ptr(idx),
                                      _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_attn_decode_asm")
    return out, lse, idx


def kv_evict_to_budget(cache: KVCache, t, M: int, evicted_pos=None, n_evicted=None, ws=None,
                       stream=None):
    """Evict every head over budget to M slots and compact in place.

    evicted_pos: optional int32 [B][Hkv][max_evict] tensor (ascending positions).
    Returns n_evicted [B][Hkv] int32 (allocated if not given).
    """
    _need(t, "t", torch.int32)
    if n_evicted is None:
        n_evicted = torch.empty((cache.B, cache.Hkv), dtype=torch.int32, device=t.device)
    _need(n_evicted, "n_evicted", torch.int32)
    max_evict = 0
    if evicted_pos is not None:
        _need(evicted_pos, "evicted_pos", torch.int32)
        max_evict = evicted_pos.shape[-1]
    ws = _ws(ws, kv_evict_workspace(cache, M), t.device)
    st = library().kv_evict_to_budget(cache.desc, _ptr(t), int(M), _ptr(evicted_pos), max_evict,
                                      _ptr(n_evicted), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_evict_to_budget")
    return n_evicted


CHECK_BITS = {"len": 1, "start": 2, "pos_order": 4, "pos_after_t": 8, "log_beta_nan": 16,
              "log_beta_positive": 32, "ranges": 64, "pages": 128}


def kv_check_pages(cache: KVCache, pages: "KVPages", t=None, flags=None, stream=None):
    """Device-side precondition check of a paged cache (kv_check_pages in kvbound.h).
    Returns the [B][Hkv] int32 tensor of violation bits (CHECK_BITS); 0 means none."""
    if t is not None:
        _need(t, "t", torch.int32)
    if flags is None:
        flags = torch.empty((cache.B, cache.Hkv), dtype=torch.int32, device=cache.pos.device)
    _need(flags, "flags", torch.int32)
    st = library().kv_check_pages(cache.desc, pages.desc, _ptr(t), _ptr(flags), _stream(stream))
    _check(st, "kv_check_pages")
    return flags


def kv_check_cache(cache: KVCache, t=None, ranges=None, n_ranges=None, flags=None,
                   stream=None):
    """Device-side precondition check (kv_check_cache in kvbound.h).  Returns the
    [B][Hkv] int32 tensor of violation bits (CHECK_BITS); 0 means none."""
    if t is not None:
        _need(t, "t", torch.int32)
    R = 0
    if n_ranges is not None:
        _need(n_ranges, "n_ranges", torch.int32)
        _need(ranges, "ranges", torch.int32)
        R = ranges.shape[1]
    if flags is None:
        flags = torch.empty((cache.B, cache.Hkv), dtype=torch.int32, device=cache.pos.device)
    _need(flags, "flags", torch.int32)
    st = library().kv_check_cache(cache.desc, _ptr(t), _ptr(ranges), _ptr(n_ranges), int(R),
                                  _ptr(flags), _stream(stream))
    _check(st, "kv_check_cache")
    return flags


def kv_append(cache: KVCache, k_new, v_new, log_beta_new, t, ws=None, stream=None,
              check_status: bool = False):
    """Append one token per KV head (slot len, pos = t[b]); len += 1.
    check_status: wait for the call and raise if a head was full."""
    _need(k_new, "k_new", cache.k.dtype)
    _need(v_new, "v_new", cache.k.dtype)
    _need(t, "t", torch.int32)
    if log_beta_new is not None:
        _need(log_beta_new, "log_beta_new", torch.float32)
    ws = _ws(ws, 256, t.device)
    st = library().kv_append(cache.desc, _ptr(k_new), _ptr(v_new), _ptr(log_beta_new), _ptr(t),
                             _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_append")
    if check_status:
        _check_ws(ws, stream, "kv_append (device status)")


def kv_evict_plan(cache: KVCache, t, M: int, evicted_pos=None, n_evicted=None, ws=None,
                  stream=None):
    """Phase 1 of eviction (reads the cache only).  Returns (n_evicted, ws); pass the
    same ws to kv_evict_apply."""
    _need(t, "t", torch.int32)
    if n_evicted is None:
        n_evicted = torch.empty((cache.B, cache.Hkv), dtype=torch.int32, device=t.device)
    max_evict = 0
    if evicted_pos is not None:
        _need(evicted_pos, "evicted_pos", torch.int32)
        max_evict = evicted_pos.shape[-1]
    ws = _ws(ws, kv_evict_workspace(cache, M), t.device)
    st = library().kv_evict_plan(cache.desc, _ptr(t), int(M), _ptr(evicted_pos), max_evict,
                                 _ptr(n_evicted), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_evict_plan")
    return n_evicted, ws


def kv_evict_apply(cache: KVCache, M: int, ws, stream=None):
    """Phase 2 of eviction: move the kept rows and set len."""
    _need(ws, "ws", torch.uint8)
    st = library().kv_evict_apply(cache.desc, int(M), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_evict_apply")


def kv_evict_one(cache: KVCache, t, M: int, evicted_pos=None, n_evicted=None, stream=None):
    """Eviction for heads at most one token over budget M (see kv_evict_one in
    kvbound.h): one launch, no workspace.  Returns n_evicted [B][Hkv] int32 (1, 0,
    or -(n - M) for a head left untouched because it is further over)."""
    _need(t, "t", torch.int32)
    B, H = cache.length.shape
    if n_evicted is None:
        n_evicted = torch.empty((B, H), dtype=torch.int32, device=t.device)
    _need(n_evicted, "n_evicted", torch.int32)
    me = 0
    if evicted_pos is not None:
        _need(evicted_pos, "evicted_pos", torch.int32)
        me = evicted_pos.shape[-1]
    st = library().kv_evict_one(cache.desc, _ptr(t), int(M), _ptr(evicted_pos), me,
                                _ptr(n_evicted), _stream(stream))
    _check(st, "kv_evict_one")
    return n_evicted


def kv_evict_one_workspace(cache: KVCache, num_splits: int = 0) -> int:
    return int(library().kv_evict_one_workspace(cache.desc, int(num_splits)))


def kv_attn_decode_evict_one_workspace(cache: KVCache, Hq: int, num_splits: int = 0) -> int:
    return int(library().kv_attn_decode_evict_one_workspace(cache.desc, int(Hq),
                                                            int(num_splits)))


def kv_attn_decode_evict_one(cache: KVCache, q, t, M: int, scale: float = 0.0, k_new=None,
                             v_new=None, log_beta_new=None, num_splits: int = 0, out=None,
                             lse=None, evicted_pos=None, n_evicted=None, ws=None, stream=None):
    """Attention with the decode token, then every head at M + 1 evicts its lowest
    token and the decode token takes that slot (see kvbound.h).  Returns (out, lse,
    n_evicted)."""
    _need(q, "q", cache.k.dtype)
    _need(t, "t", torch.int32)
    B, Hq, D = q.shape
    H = cache.length.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if n_evicted is None:
        n_evicted = torch.empty((B, H), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _need(n_evicted, "n_evicted", torch.int32)
    me = 0
    if evicted_pos is not None:
        _need(evicted_pos, "evicted_pos", torch.int32)
        me = evicted_pos.shape[-1]
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x is not None:
            _need(x, name, cache.k.dtype)
    if log_beta_new is not None:
        _need(log_beta_new, "log_beta_new", torch.float32)
    ws = _ws(ws, kv_attn_decode_evict_one_workspace(cache, Hq, num_splits), q.device)
    st = library().kv_attn_decode_evict_one(
        cache.desc, _ptr(q), Hq, _ptr(t), float(scale), _ptr(k_new), _ptr(v_new),
        _ptr(log_beta_new), int(M), int(num_splits), _ptr(out), _ptr(lse), _ptr(evicted_pos),
        me, _ptr(n_evicted), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_attn_decode_evict_one")
    return out, lse, n_evicted


def kv_attn_decode_plan_one(cache: KVCache, q, t, ws_evict, scale: float = 0.0, k_new=None,
                            v_new=None, log_beta_new=None, num_splits: int = 0, out=None,
                            lse=None, ws=None, stream=None):
    """kv_attn_decode that also plans each head's one-token eviction (order-keeping
    shift) in ws_evict (kv_evict_one_workspace bytes) for kv_evict_one_apply.
    Returns (out, lse)."""
    _need(q, "q", cache.k.dtype)
    _need(t, "t", torch.int32)
    _need(ws_evict, "ws_evict")
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x is not None:
            _need(x, name, cache.k.dtype)
    if log_beta_new is not None:
        _need(log_beta_new, "log_beta_new", torch.float32)
    ws = _ws(ws, kv_attn_decode_workspace(cache, Hq, num_splits), q.device)
    st = library().kv_attn_decode_plan_one(
        cache.desc, _ptr(q), Hq, _ptr(t), float(scale), _ptr(k_new), _ptr(v_new),
        _ptr(log_beta_new), int(num_splits), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
        _ptr(ws_evict), ws_evict.numel() * ws_evict.element_size(), _stream(stream))
    _check(st, "kv_attn_decode_plan_one")
    return out, lse


def kv_evict_one_apply(cache: KVCache, t, M: int, ws_evict, evicted_pos=None, n_evicted=None,
                       stream=None):
    """The eviction kv_attn_decode_plan_one planned (see kvbound.h): heads at M + 1
    lose their lowest-retention token, the rows keeping position order.  Returns
    n_evicted [B][Hkv] int32 (1, 0, or -(n - M) for a head left untouched)."""
    _need(t, "t", torch.int32)
    _need(ws_evict, "ws_evict")
    B, H = cache.length.shape
    if n_evicted is None:
        n_evicted = torch.empty((B, H), dtype=torch.int32, device=t.device)
    _need(n_evicted, "n_evicted", torch.int32)
    me = 0
    if evicted_pos is not None:
        _need(evicted_pos, "evicted_pos", torch.int32)
        me = evicted_pos.shape[-1]
    st = library().kv_evict_one_apply(cache.desc, _ptr(t), int(M), _ptr(evicted_pos), me,
                                      _ptr(n_evicted), _ptr(ws_evict),
                                      ws_evict.numel() * ws_evict.element_size(),
                                      _stream(stream))
    _check(st, "kv_evict_one_apply")
    return n_evicted


def kv_attn_decode_compact(cache: KVCache, q, t, M: int, ws_evict, scale: float = 0.0,
                           num_splits: int = 0, phase: int = 0, out=None, lse=None, ws=None,
                           stream=None):
    """Attention + the planned compaction in one pass (plan: kv_evict_plan with the
    same M and ws_evict).  phase 0 = all; 1 = first tiles only; 2 = the rest.
    Returns (out, lse)."""
    _need(q, "q", cache.k.dtype)
    _need(t, "t", torch.int32)
    _need(ws_evict, "ws_evict", torch.uint8)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws = _ws(ws, kv_attn_decode_workspace(cache, Hq, num_splits), q.device)
    st = library().kv_attn_decode_compact(cache.desc, _ptr(q), Hq, _ptr(t), float(scale), int(M),
                                          int(num_splits), int(phase), _ptr(out), _ptr(lse),
                                          _ptr(ws), ws.numel(), _ptr(ws_evict), ws_evict.numel(),
                                          _stream(stream))
    _check(st, "kv_attn_decode_compact")
    return out, lse


def kv_erase_ranges(cache: KVCache, ranges, n_ranges, n_erased=None, ws=None, stream=None):
    """Erase half-open position ranges ([B][R][2] int32) from every head; compact in place."""
    _need(ranges, "ranges", torch.int32)
    _need(n_ranges, "n_ranges", torch.int32)
    if ranges.dim() != 3 or ranges.shape[-1] != 2:
        raise ValueError("ranges must be [B][R][2]")
    if n_erased is None:
        n_erased = torch.empty((cache.B, cache.Hkv), dtype=torch.int32, device=ranges.device)
    ws = _ws(ws, kv_erase_workspace(cache), ranges.device)
    st = library().kv_erase_ranges(cache.desc, _ptr(ranges), _ptr(n_ranges), ranges.shape[1],
                                   _ptr(n_erased), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kv_erase_ranges")
    return n_erased


def kv_attn_decode_paged(cache: KVCache, pages: KVPages, q, t, scale: float = 0.0, k_new=None,
                         v_new=None, log_beta_new=None, spare=None, num_splits: int = 0,
                         out=None, lse=None, ws=None, stream=None, check_status: bool = False):
    """kv_attn_decode over a paged cache; the decode token (optional) goes into the
    last page, or the free page spare [B][Hkv] int32.  Returns (out, lse)."""
    _need(q, "q", cache.k.dtype)
    _need(t, "t", torch.int32)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x is not None:
            _need(x, name, cache.k.dtype)
    if log_beta_new is not None:
        _need(log_beta_new, "log_beta_new", torch.float32)
    if spare is not None:
        _need(spare, "spare", torch.int32)
    ws = _ws(ws, kv_attn_decode_workspace(cache, Hq, num_splits), q.device)
    st = library().kv_attn_decode_paged(cache.desc, pages.desc, _ptr(q), Hq, _ptr(t),
                                        float(scale), _ptr(k_new), _ptr(v_new),
                                        _ptr(log_beta_new), _ptr(spare), int(num_splits),
                                        _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                        _stream(stream))
    _check(st, "kv_attn_decode_paged")
    if check_status:
        _check_ws(ws, stream, "kv_attn_decode_paged (device status)")
    return out, lse


def kv_erase_paged_workspace(cache: KVCache, pages: KVPages) -> int:
    return int(library().kv_erase_paged_workspace(cache.desc, pages.desc))


def kv_erase_ranges_paged(cache: KVCache, pages: KVPages, ranges, n_ranges, n_erased=None,
                          ws=None, stream=None):
    """Block-granular erase of half-open position ranges ([B][R][2] int32) over a
    paged cache: fully erased pages leave the table, partial pages compact in place."""
    _need(ranges, "ranges", torch.int32)
    _need(n_ranges, "n_ranges", torch.int32)
    if ranges.dim() != 3 or ranges.shape[-1] != 2:
        raise ValueError("ranges must be [B][R][2]")
    if n_erased is None:
        n_erased = torch.empty((cache.B, cache.Hkv), dtype=torch.int32, device=ranges.device)
    ws = _ws(ws, kv_erase_paged_workspace(cache, pages), ranges.device)
    st = library().kv_erase_ranges_paged(cache.desc, pages.desc, _ptr(ranges), _ptr(n_ranges),
                                         ranges.shape[1], _ptr(n_erased), _ptr(ws), ws.numel(),
                                         _stream(stream))
    _check(st, "kv_erase_ranges_paged")
    return n_erased


def asm_lookup_merge(q, centroids, abar, log_zbar, self_out, self_lse, out=None, out_lse=None,
                     idx=None, ws=None, stream=None):
    """Cosine-argmax codebook lookup + merge with the query's own state.

    Returns (out, out_lse, idx).
    """
    _need(q, "q", torch.bfloat16)
    _need(centroids, "centroids", torch.bfloat16)
    _need(abar, "abar", torch.bfloat16)
    _need(log_zbar, "log_zbar", torch.float32)
    _need(self_out, "self_out", torch.float32)
    _need(self_lse, "self_lse", torch.float32)
    B, Hq, D = q.shape
    Hkv, K, D2 = centroids.shape
    if D2 != D or tuple(abar.shape) != (Hkv, K, D) or tuple(log_zbar.shape) != (Hkv, K):
        raise ValueError("codebook shapes must be [Hkv][K][D] and [Hkv][K]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    ws = _ws(ws, asm_lookup_merge_workspace(B, Hq, Hkv, D, K), q.device)
    st = library().asm_lookup_merge(_ptr(q), B, Hq, Hkv, D, _ptr(centroids), _ptr(abar),
                                    _ptr(log_zbar), K, _ptr(self_out), _ptr(self_lse), _ptr(out),
                                    _ptr(out_lse), _ptr(idx), _ptr(ws), ws.numel(),
                                    _stream(stream))
    _check(st, "asm_lookup_merge")
    return out, out_lse, idx


TRACE_BITS = {"attn_split": 1, "attn_merge": 2, "append": 4, "evict_select": 8,
              "keep_count": 16, "keep_emit": 32, "compact_move": 64, "asm_lookup": 128,
              "asm_finalize": 256, "attn_fused": 512, "asm_prefix": 1024,
              "asm_prefix_merge": 2048, "km_assign": 4096, "km_update": 8192,
              "asm_aggregate": 16384, "asm_vt": 32768, "latent_absorb": 65536,
              "latent_read": 131072, "evict_one": 262144, "erase_search": 524288,
              "erase_plan": 1048576, "one_shift": 4194304,
              "erase_pages": 8388608}


def asm_lookup_merge_hier_workspace(B, Hq, Hkv, K1, m) -> int:
    return int(library().asm_lookup_merge_hier_workspace(B, Hq, Hkv, K1, m))


def asm_lookup_merge_hier(q, c1, offs, centroids, kid, m, abar, log_zbar, self_out, self_lse,
                          out=None, out_lse=None, idx=None, ws=None, stream=None):
    """Two-level lookup + merge (see asm_lookup_merge_hier in kvbound.h).
    c1 [Hkv][K1][D], offs [Hkv][K1+1], centroids (cluster order) [Hkv][K][D],
    kid [Hkv][K]; abar, log_zbar by original index.  Returns (out, out_lse, idx)."""
    _need(q, "q", torch.bfloat16)
    _need(c1, "c1", torch.bfloat16)
    _need(offs, "offs", torch.int32)
    _need(centroids, "centroids", torch.bfloat16)
    _need(kid, "kid", torch.int32)
    _need(abar, "abar", torch.bfloat16)
    _need(log_zbar, "log_zbar", torch.float32)
    _need(self_out, "self_out", torch.float32)
    _need(self_lse, "self_lse", torch.float32)
    B, Hq, D = q.shape
    Hkv, K1, _ = c1.shape
    K = centroids.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    ws = _ws(ws, asm_lookup_merge_hier_workspace(B, Hq, Hkv, K1, m), q.device)
    st = library().asm_lookup_merge_hier(_ptr(q), B, Hq, Hkv, D, _ptr(c1), K1, _ptr(offs),
                                         _ptr(centroids), _ptr(kid), K, int(m), _ptr(abar),
                                         _ptr(log_zbar), _ptr(self_out), _ptr(self_lse), _ptr(out),
                                         _ptr(out_lse), _ptr(idx), _ptr(ws), ws.numel(),
                                         _stream(stream))
    _check(st, "asm_lookup_merge_hier")
    return out, out_lse, idx


def trace_enable(capacity: int, kernels=("attn_split",)):
    """Record HIP event pairs around the named kernels' launches (see kvb_trace_enable)."""
    mask = 0
    for k in kernels:
        mask |= TRACE_BITS[k]
    _check(library().kvb_trace_enable(int(capacity), mask), "kvb_trace_enable")


def trace_read(max_entries: int = 1 << 16):
    """[(kernel name, milliseconds)] for every recorded launch (waits for them)."""
    import numpy as np
    ids = np.zeros(max_entries, np.int32)
    ms = np.zeros(max_entries, np.float32)
    n = library().kvb_trace_read(ids.ctypes.data_as(ctypes.c_void_p),
                                 ms.ctypes.data_as(ctypes.c_void_p), max_entries)
    names = {v: k for k, v in TRACE_BITS.items()}
    return [(names.get(int(i), str(int(i))), float(m)) for i, m in zip(ids[:n], ms[:n])]


def trace_reset():
    library().kvb_trace_reset()


def trace_disable():
    library().kvb_trace_disable()


def asm_prefix_states_workspace(H, N, D, L, chunks) -> int:
    return int(library().asm_prefix_states_workspace(H, N, D, L, chunks))


def asm_kmeans_workspace(H, K, D) -> int:
    return int(library().asm_kmeans_workspace(H, K, D))


def asm_build_memory_workspace(H, N, D, L, chunks, K) -> int:
    return int(library().asm_build_memory_workspace(H, N, D, L, chunks, K))


def _prefix_shapes(q, k, v):
    _need(q, "q", torch.bfloat16)
    H, N, D = q.shape
    if k is None or v is None:
        raise ValueError("k and v are required (shape [H][0][D] for an empty prefix)")
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16)
    if k.dim() != 3 or tuple(k.shape) != tuple(v.shape) or k.shape[0] != H or k.shape[2] != D:
        raise ValueError("k, v must be [H][L][D] matching q [H][N][D]")
    return H, N, D, k.shape[1]


def asm_prefix_states(q, k, v, chunks: int = 1, scale: float = 0.0, a=None, lse=None, ws=None,
                      stream=None):
    """States (a [H][N][D] f32, lse [H][N] f32) of the queries q [H][N][D] over the
    prefix k, v [H][L][D], computed in `chunks` chunks and merged."""
    H, N, D, L = _prefix_shapes(q, k, v)
    if a is None:
        a = torch.empty((H, N, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    _need(a, "a", torch.float32)
    _need(lse, "lse", torch.float32)
    ws = _ws(ws, asm_prefix_states_workspace(H, N, D, L, chunks), q.device)
    st = library().asm_prefix_states(_ptr(q), H, N, D, _ptr(k), _ptr(v), L, int(chunks),
                                     float(scale), _ptr(a), _ptr(lse), _ptr(ws), ws.numel(),
                                     _stream(stream))
    _check(st, "asm_prefix_states")
    return a, lse


def asm_kmeans(x, centroids, iters: int, assign=None, counts=None, centroids_bf16=None, ws=None,
               stream=None):
    """Lloyd K-means of x [H][N][D] bf16 from centroids [H][K][D] f32 (updated in
    place).  Returns (assign [H][N] i32, counts [H][K] i32, centroids_bf16 or None)."""
    _need(x, "x", torch.bfloat16)
    _need(centroids, "centroids", torch.float32)
    H, N, D = x.shape
    if centroids.dim() != 3 or centroids.shape[0] != H or centroids.shape[2] != D:
        raise ValueError("centroids must be [H][K][D] matching x [H][N][D]")
    K = centroids.shape[1]
    if assign is None:
        assign = torch.empty((H, N), dtype=torch.int32, device=x.device)
    if counts is None:
        counts = torch.empty((H, K), dtype=torch.int32, device=x.device)
    _need(assign, "assign", torch.int32)
    _need(counts, "counts", torch.int32)
    if centroids_bf16 is not None:
        _need(centroids_bf16, "centroids_bf16", torch.bfloat16)
    ws = _ws(ws, asm_kmeans_workspace(H, K, D), x.device)
    st = library().asm_kmeans(_ptr(x), H, N, D, _ptr(centroids), K, int(iters), _ptr(assign),
                              _ptr(counts), _ptr(centroids_bf16), _ptr(ws), ws.numel(),
                              _stream(stream))
    _check(st, "asm_kmeans")
    return assign, counts, centroids_bf16


def asm_aggregate_states(assign, a, lse, K: int, abar=None, log_zbar=None, stream=None):
    """Per cluster the merge of its members' states.  Returns (abar [H][K][D] bf16,
    log_zbar [H][K] f32)."""
    _need(assign, "assign", torch.int32)
    _need(a, "a", torch.float32)
    _need(lse, "lse", torch.float32)
    H, N, D = a.shape
    if tuple(assign.shape) != (H, N) or tuple(lse.shape) != (H, N):
        raise ValueError("assign and lse must be [H][N] matching a [H][N][D]")
    if abar is None:
        abar = torch.empty((H, K, D), dtype=torch.bfloat16, device=a.device)
    if log_zbar is None:
        log_zbar = torch.empty((H, K), dtype=torch.float32, device=a.device)
    _need(abar, "abar", torch.bfloat16)
    _need(log_zbar, "log_zbar", torch.float32)
    st = library().asm_aggregate_states(_ptr(assign), _ptr(a), _ptr(lse), H, N, D, int(K),
                                        _ptr(abar), _ptr(log_zbar), _stream(stream))
    _check(st, "asm_aggregate_states")
    return abar, log_zbar


def asm_build_memory(q, k, v, centroids, iters: int, chunks: int = 1, scale: float = 0.0,
                     centroids_bf16=None, abar=None, log_zbar=None, assign=None, ws=None,
                     stream=None):
    """Offline memory build for one layer: prefix states, K-means, aggregation.
    centroids [H][K][D] f32 holds the initial centroids and is updated in place.
    Returns (centroids_bf16, abar, log_zbar, assign, ws); ws holds the states."""
    H, N, D, L = _prefix_shapes(q, k, v)
    _need(centroids, "centroids", torch.float32)
    if centroids.dim() != 3 or centroids.shape[0] != H or centroids.shape[2] != D:
        raise ValueError("centroids must be [H][K][D] matching q [H][N][D]")
    K = centroids.shape[1]
    dev = q.device
    if centroids_bf16 is None:
        centroids_bf16 = torch.empty((H, K, D), dtype=torch.bfloat16, device=dev)
    if abar is None:
        abar = torch.empty((H, K, D), dtype=torch.bfloat16, device=dev)
    if log_zbar is None:
        log_zbar = torch.empty((H, K), dtype=torch.float32, device=dev)
    if assign is None:
        assign = torch.empty((H, N), dtype=torch.int32, device=dev)
    _need(centroids_bf16, "centroids_bf16", torch.bfloat16)
    _need(abar, "abar", torch.bfloat16)
    _need(log_zbar, "log_zbar", torch.float32)
    _need(assign, "assign", torch.int32)
    ws = _ws(ws, asm_build_memory_workspace(H, N, D, L, chunks, K), dev)
    st = library().asm_build_memory(_ptr(q), H, N, D, _ptr(k), _ptr(v), L, int(chunks),
                                    float(scale), _ptr(centroids), K, int(iters),
                                    _ptr(centroids_bf16), _ptr(abar), _ptr(log_zbar),
                                    _ptr(assign), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "asm_build_memory")
    return centroids_bf16, abar, log_zbar, assign, ws


def kv_latent_absorb_workspace(cache: KVCache) -> int:
    return int(library().kv_latent_absorb_workspace(cache.desc))


def kv_latent_absorb(cache: KVCache, M: int, ws_evict, lam: float, mem_M, mem_b, ws=None,
                     stream=None):
    """Absorb the tokens the plan in ws_evict evicts into the latent memory (mem_M
    [B][Hkv][D][D], mem_b [B][Hkv][D], float32, updated in place).  Call between
    kv_evict_plan and kv_evict_apply."""
    _need(ws_evict, "ws_evict", torch.uint8)
    _need(mem_M, "mem_M", torch.float32)
    _need(mem_b, "mem_b", torch.float32)
    D = cache.D
    if tuple(mem_M.shape) != (cache.B, cache.Hkv, D, D) or tuple(mem_b.shape) != (cache.B,
                                                                                   cache.Hkv, D):
        raise ValueError("mem_M must be [B][Hkv][D][D], mem_b [B][Hkv][D]")
    ws = _ws(ws, kv_latent_absorb_workspace(cache), mem_M.device)
    st = library().kv_latent_absorb(cache.desc, int(M), _ptr(ws_evict), ws_evict.numel(),
                                    float(lam), _ptr(mem_M), _ptr(mem_b), _ptr(ws), ws.numel(),
                                    _stream(stream))
    _check(st, "kv_latent_absorb")


def kv_latent_read(q, mem_M, mem_b, W_o, w_g, c_g, eps: float, out, stream=None):
    """out [B][Hq][D] (float32, holding o_attn) += g(q) m(q) from the latent memory."""
    _need(q, "q", torch.bfloat16)
    for name, x in (("mem_M", mem_M), ("mem_b", mem_b), ("W_o", W_o), ("w_g", w_g),
                    ("c_g", c_g), ("out", out)):
        _need(x, name, torch.float32)
    B, Hq, D = q.shape
    Hkv = mem_M.shape[1]
    if (tuple(mem_M.shape) != (B, Hkv, D, D) or tuple(mem_b.shape) != (B, Hkv, D)
            or tuple(W_o.shape) != (D, D) or tuple(w_g.shape) != (Hq, D)
            or tuple(c_g.shape) != (Hq,) or tuple(out.shape) != (B, Hq, D)):
        raise ValueError("latent read shapes")
    st = library().kv_latent_read(_ptr(q), B, Hq, Hkv, D, _ptr(mem_M), _ptr(mem_b), _ptr(W_o),
                                  _ptr(w_g), _ptr(c_g), float(eps), _ptr(out), _stream(stream))
    _check(st, "kv_latent_read")
    return out
