"""Chunked-prefill attention over the paged cache, as plain float64 NumPy.

Test infrastructure only (see the package docstring).

Prefill handles a prompt's query positions together, as matrix products
(page "KV Cache and Inference Optimization", the prefill / decode comparison;
page "Understanding KV Cache" §2.1). Split into chunks, a chunk's K/V rows are
appended to the cache first; each of its query tokens then attends causally to
every cached position up to its own (§1.2: position i sees positions <= i).
Token i of a chunk of q_len tokens whose sequence holds n cached tokens (the
chunk included) sits at position n - q_len + i, so its output is exactly the
single-query attention over the first n - q_len + i + 1 cached tokens: the
definition below gathers each sequence once and gives every query token the
prefix of that gather that its position allows.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .paged_decode import _attend_heads, gather_sequence, gather_sequence_fp8, upcast


def prefill_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                      q_start: Sequence[int], context_lens: Sequence[int], scale: float, num_kv_heads: int,
                      block_size: int, dtype: str, layout: str = "HND") -> np.ndarray:
    """q: [total_q, Hq, D] raw; sequence b's chunk is rows q_start[b]..q_start[b+1]-1.
    Returns float64 [total_q, Hq, D]."""
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(len(context_lens)):
        q0, q1 = int(q_start[b]), int(q_start[b + 1])
        n = int(context_lens[b])
        q_len = min(q1 - q0, n)
        if q_len <= 0:
            continue
        K = [gather_sequence(k_cache, dtype, block_tables[b], n, j, block_size, layout) for j in range(num_kv_heads)]
        V = [gather_sequence(v_cache, dtype, block_tables[b], n, j, block_size, layout) for j in range(num_kv_heads)]
        for i in range(q_len):
            m = n - q_len + i + 1  # keys at positions 0 .. n - q_len + i
            out[q0 + i] = _attend_heads(upcast(q[q0 + i], dtype), lambda j: K[j][:m], lambda j: V[j][:m],
                                        num_kv_heads, m, scale)
    return out


def prefill_attention_fp8(q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray,
                          v_scales: np.ndarray, block_tables: np.ndarray, q_start: Sequence[int],
                          context_lens: Sequence[int], scale: float, num_kv_heads: int, block_size: int,
                          q_dtype: str, layout: str = "HND", fmt: str = "e4m3") -> np.ndarray:
    """As ``prefill_attention`` over 8-bit caches (values decode(code) * scale,
    codes in format ``fmt``)."""
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(len(context_lens)):
        q0, q1 = int(q_start[b]), int(q_start[b + 1])
        n = int(context_lens[b])
        q_len = min(q1 - q0, n)
        if q_len <= 0:
            continue
        row = block_tables[b]
        K = [gather_sequence_fp8(k_codes, k_scales, row, n, j, block_size, layout, fmt) for j in range(num_kv_heads)]
        V = [gather_sequence_fp8(v_codes, v_scales, row, n, j, block_size, layout, fmt) for j in range(num_kv_heads)]
        for i in range(q_len):
            m = n - q_len + i + 1
            out[q0 + i] = _attend_heads(upcast(q[q0 + i], q_dtype), lambda j: K[j][:m], lambda j: V[j][:m],
                                        num_kv_heads, m, scale)
    return out
