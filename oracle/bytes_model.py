"""KV-cache byte counts (the unit of the HBM roofline).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The IndexMem page (technical summary, section 1, problem statement) estimates
about 320 GB of KV cache for a 70B-parameter model at a one-million-token
context.  K and V each hold head_dim values per KV head per layer per token,
which with an 80-layer, 8-KV-head, head_dim-128 model in 2-byte storage gives
exactly 320 GiB at 2^20 tokens; that architecture is an assumption consistent
with the figure (the page does not give it).
"""
from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of K plus V for one token across all layers and KV heads."""
    return 2 * layers * kv_heads * head_dim * elem_bytes

