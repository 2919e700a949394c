"""KV-cache byte and block accounting, written out from the pages' closed forms.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

from typing import Iterable


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int,
                   tokens: int, seqs: int) -> int:
    """KV bytes = 2 x L x Hkv x D x B x T x N.

    Page "Why does a request use more memory the longer it generates?"
    (learning-field-guides.pages.dev, 06-inference), section "Deriving capacity
    from the K and V dimensions": K and V (the factor 2) for each of L layers,
    Hkv KV heads, D elements per head of B bytes each, T positions and N
    sequences. The same product is the "KV Cache Size" formula of §1.4 of the
    page "Understanding KV Cache" (steinslab.io) with seqs = 1.
    """
    return 2 * layers * kv_heads * head_dim * bytes_per_elem * tokens * seqs


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    """bytes_per_token = 2 x layers x kv_heads x head_dim x bytes_per_element.

    Page "KV Cache and Inference Optimization" (note.yj-dis.top), section
    "How big is the KV cache: a memory bill".
    """
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def ragged_kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int,
                          lengths: Iterable[int]) -> int:
    """Ragged batch: T x N replaced by the sum of the per-sequence lengths.

    Page "Why does a request use more memory the longer it generates?",
    section "Paging changes allocation, not a token's representation" (the
    closing paragraph on unequal request lengths).
    """
    return 2 * layers * kv_heads * head_dim * bytes_per_elem * sum(int(t) for t in lengths)


def block_bytes(kv_heads: int, block_size: int, head_dim: int, bytes_per_elem: int) -> int:
    """One layer's block of logical shape [2, num_kv_heads, block_size, head_dim].

    Page "Understanding KV Cache" (steinslab.io), §3.2 "Physical layout of a
    block" (HND layout).
    """
    return 2 * kv_heads * block_size * head_dim * bytes_per_elem


def blocks_for(positions: int, block_size: int) -> int:
    """Blocks a sequence of ``positions`` cached positions occupies: ceil(n / bs).

    Page "Why does a request use more memory...", section "Paging changes
    allocation" (18 positions in 16-slot blocks need two blocks).
    """
    if positions < 0 or block_size <= 0:
        raise ValueError("positions must be >= 0 and block_size > 0")
    return (positions + block_size - 1) // block_size


def block_capacity(positions: int, block_size: int) -> int:
    """Positions the allocated blocks can hold (blocks x block size)."""
    return blocks_for(positions, block_size) * block_size


def empty_slots(positions: int, block_size: int) -> int:
    """Empty positions left in the last block (internal fragmentation).

    Same section as ``blocks_for``; also the page "The KV Cache Problem of
    Traditional Attention" (pyllm.pages.dev), §1.3, "Internal fragmentation"
    with a 256-token allocation unit.
    """
    return block_capacity(positions, block_size) - positions
