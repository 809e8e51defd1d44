"""Plain float64 CPU oracle for bounded decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product.

Every function is a direct, unblocked statement of what the pages define:

* ``attention``   -- retention-biased softmax attention for one decode query
  ("Cache What Lasts: Token Retention for Memory-Bounded KV Cache in LLMs",
  section 2.1, retention-gated attention) with the 1/sqrt(d) dot-product scale of
  "Context Memorization for Efficient Long Context Generation" (method steps,
  step 1), and the attention state (a, Z) of the latter page.
* ``merge``       -- the attention-state merge operator (Context Memorization,
  method steps, step 2 and step 4; the online-softmax identity in the
  background-knowledge section).
* ``eviction``    -- TRIM-KV inference-time eviction of the lowest retention
  score beta_i^(t-i) when a head exceeds its budget M ("Cache What Lasts",
  section 2.2, inference), followed by an order-preserving compaction.
* ``erase``       -- MEMENTO's in-place removal of thinking-block entries
  ("MEMENTO: Teaching LLMs to Manage Their Own Context", blocks-and-compression
  section and the systems section on the modified engine).
* ``asm``         -- cosine-argmax centroid lookup and lossless state merge
  (Context Memorization, method steps, steps 3 and 4; GQA extension in the
  technical-novelty section), and the two-level (hierarchical) lookup of the
  same section.
* ``asm_build``   -- construction of that memory: prefix attention states of
  calibration queries (chunked and merged), K-means over the queries, and the
  merge of each cluster's states (Context Memorization, method steps 1 and 2).
* ``latent``      -- IndexMem's latent memory of evicted tokens: decayed
  outer-product fast weights (M, b) and the gated residual read-out ("IndexMem:
  Learned KV-Cache Eviction with Latent Memory for Long-Context LLM Inference",
  technical summary, section 2, part B).
* ``decode``      -- the decode loop (append, attend, evict) of "Cache What
  Lasts", section 2.2 (inference).
* ``bytes_model`` -- KV bytes per token, pinned to IndexMem's memory-wall figure
  ("IndexMem: Learned KV-Cache Eviction with Latent Memory for Long-Context LLM
  Inference", technical summary, section 1).

Readings taken where the pages are silent are stated in each function's
docstring.  Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (identities, closed forms, brute force and a
library routine), and ``tests/test_oracle_mutations.py`` shows that planted
mistakes fail those pins.
"""
from .attn import (retention_bias, attention_state, attention, merge_states,
                        state_to_out_lse, split_attention, decode_attention)
from .evict import (retention_keys, evict_plan, erase_plan, compact_unit,
                       Cache, evict_to_budget, erase_ranges, append_tokens)
from .asm import (cosine_similarities, cosine_lookup, asm_merge, asm_lookup_merge,
                  hier_lookup, asm_lookup_merge_hier)
from .asm_build import (chunk_bounds, prefix_states, nearest_centroid, centroid_update,
                        kmeans, aggregate_states, build_memory)
from .bytes_model import kv_bytes_per_token
from .latent import phi, latent_absorb, latent_read, latent_residual
from .decode import run_decode_steps

__all__ = [
    "retention_bias", "attention_state", "attention", "merge_states",
    "state_to_out_lse", "split_attention", "decode_attention",
    "retention_keys", "evict_plan", "erase_plan", "compact_unit", "Cache",
    "evict_to_budget", "erase_ranges", "append_tokens",
    "cosine_similarities", "cosine_lookup", "asm_merge", "asm_lookup_merge",
    "hier_lookup", "asm_lookup_merge_hier",
    "chunk_bounds", "prefix_states", "nearest_centroid", "centroid_update", "kmeans",
    "aggregate_states", "build_memory",
    "kv_bytes_per_token", "run_decode_steps",
    "phi", "latent_absorb", "latent_read", "latent_residual",
]
