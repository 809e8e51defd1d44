"""Python binding of libkvbound (decode attention over a memory-bounded KV cache).

Argument marshalling only: every step runs in the HIP library's kernels.  Torch
tensors supply device memory and the current stream.  The library must be built
(``python -m bounded_decode_attention_amd.build``); importing this module does
not build it, and every call fails loudly if it is missing.

Entry points (same names as the C ABI in include/kvbound.h):
    kv_attn_decode, kv_evict_to_budget, kv_erase_ranges, asm_lookup_merge
(kv_attn_decode_asm: the first and the last in one call; kv_attn_decode_noalloc:
the first without a workspace, for callers that cannot allocate;
kv_attn_decode_evict_one, and kv_attn_decode_plan_one + kv_evict_one_apply: the
steady state's attention with the one-token eviction selected by its splits;
kv_attn_decode_paged and kv_erase_ranges_paged: the attention and the
block-granular erase over a paged cache, ``KVPages``), and, for building the
memory asm_lookup_merge reads, asm_prefix_states,
asm_kmeans, asm_aggregate_states, asm_build_memory; and the latent memory of
evicted tokens, kv_latent_absorb and kv_latent_read;
plus the workspace-size helpers and ``KVCache``, a holder of one layer's tensors.
"""
from ._lib import (KVBError, KVCache, asm_aggregate_states, asm_build_memory,
                   asm_build_memory_workspace, asm_kmeans, asm_kmeans_workspace,
                   asm_lookup_merge, asm_lookup_merge_hier, asm_prefix_states,
                   asm_prefix_states_workspace,
                   asm_lookup_merge_hier_workspace, asm_lookup_merge_workspace,
                   NOALLOC_SCRATCH_BYTES, kv_append, kv_attn_decode, kv_attn_decode_asm,
                   kv_attn_decode_asm_workspace, kv_attn_decode_asm_splits,
                   kv_attn_decode_noalloc, workspace_status,
                   kv_check_cache, kv_check_pages, CHECK_BITS,
                   kv_attn_decode_compact, kv_attn_decode_splits, kv_attn_decode_workspace,
                   kv_erase_ranges, kv_erase_workspace, kv_evict_apply, kv_evict_one,
                   kv_evict_plan, kv_attn_decode_plan_one, kv_evict_one_apply,
                   kv_evict_one_workspace, kv_attn_decode_evict_one,
                   kv_attn_decode_evict_one_workspace,
                   KVPages, kv_attn_decode_paged, kv_erase_paged_workspace,
                   kv_erase_ranges_paged,
                   kv_latent_absorb, kv_latent_absorb_workspace, kv_latent_read,
                   kv_evict_to_budget,
                   kv_evict_workspace, library, library_path, strerror, trace_disable,
                   trace_enable, trace_read, trace_reset)

__all__ = [
    "KVBError", "KVCache", "kv_attn_decode", "kv_evict_to_budget", "kv_erase_ranges",
    "kv_attn_decode_noalloc", "NOALLOC_SCRATCH_BYTES", "workspace_status",
    "kv_check_cache", "kv_check_pages", "CHECK_BITS",
    "kv_append", "kv_evict_plan", "kv_evict_apply", "kv_evict_one", "kv_attn_decode_compact",
    "kv_attn_decode_plan_one", "kv_evict_one_apply", "kv_evict_one_workspace",
    "kv_attn_decode_evict_one", "kv_attn_decode_evict_one_workspace",
    "KVPages", "kv_attn_decode_paged", "kv_erase_paged_workspace", "kv_erase_ranges_paged",
    "kv_attn_decode_asm", "kv_attn_decode_asm_workspace", "kv_attn_decode_asm_splits",
    "asm_lookup_merge", "asm_lookup_merge_hier", "asm_lookup_merge_hier_workspace",
    "kv_latent_absorb", "kv_latent_absorb_workspace", "kv_latent_read",
    "asm_prefix_states", "asm_kmeans", "asm_aggregate_states", "asm_build_memory",
    "asm_prefix_states_workspace", "asm_kmeans_workspace", "asm_build_memory_workspace",
    "kv_attn_decode_workspace", "kv_attn_decode_splits",
    "kv_evict_workspace", "kv_erase_workspace", "asm_lookup_merge_workspace",
    "library", "library_path", "strerror", "trace_enable", "trace_read", "trace_reset",
    "trace_disable",
]
