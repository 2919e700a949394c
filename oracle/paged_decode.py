"""Paged decode attention and KV append, as plain float64 NumPy.

Test infrastructure only (see the package docstring). The computation is the
plain definition: gather the sequence's cached K/V through its block table into
contiguous arrays, then run dense softmax attention for the single new query.

Storage conventions shared with the inputs (not with the GPU code):
  * caches are raw arrays of shape [num_blocks, num_kv_heads, block_size,
    head_dim] (layout "HND") or [num_blocks, block_size, num_kv_heads,
    head_dim] (layout "NHD"), the two block layouts of §3.2 of the page
    "Understanding KV Cache"; element type float32 ("f32"), float16 ("f16") or
    uint16 holding bfloat16 bits ("bf16");
  * q is [num_seqs, num_heads, head_dim], k/v of the new token are
    [num_seqs, num_kv_heads, head_dim], in the same raw storage;
  * context_lens[b] counts the tokens attended by sequence b, the newest one
    included (the query at position n-1 sees positions 0..n-1).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def upcast(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored values to float64 (every f32/f16/bf16 value
    is representable in float64)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(raw, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def slot_address(position: int, table_row: Sequence[int], block_size: int):
    """Two-level slot addressing of one token.

    Page "Understanding KV Cache" (steinslab.io), §3.3 "Slot addressing":
    logical block = floor(i / block_size), offset = i mod block_size,
    physical block = block_table[logical block], and the flat slot number is
    physical block x block_size + offset. Returns all four.
    """
    lb = position // block_size
    off = position % block_size
    pb = int(table_row[lb])
    return lb, off, pb, pb * block_size + off


def slot_mapping(block_tables: np.ndarray, positions: Sequence[int], block_size: int) -> np.ndarray:
    """Slot of each sequence's token at ``positions[b]``; a negative position
    (a padding entry) maps to slot -1, which the append skips."""
    out = np.empty(len(positions), dtype=np.int64)
    for b, pos in enumerate(positions):
        pos = int(pos)
        out[b] = -1 if pos < 0 else slot_address(pos, block_tables[b], block_size)[3]
    return out


def _at(cache: np.ndarray, pb: int, off: int, kv_head: int, layout: str):
    """Index of token `off` of block `pb`, KV head `kv_head` (the trailing axes stay)."""
    if layout == "HND":
        return cache[pb, kv_head, off]
    if layout == "NHD":
        return cache[pb, off, kv_head]
    raise ValueError(f"unknown layout {layout!r}")


def gather_sequence(cache: np.ndarray, dtype: str, table_row: Sequence[int], n: int,
                    kv_head: int, block_size: int, layout: str = "HND") -> np.ndarray:
    """Contiguous float64 [n, head_dim] copy of one KV head of one sequence.

    The attention kernel collects K/V from the physical blocks the block table
    names, in logical order (page "KV Cache and Inference Optimization",
    section "PagedAttention: manage the KV cache like virtual memory"); token i
    lives at (physical block, offset) from ``slot_address``.
    """
    head_dim = cache.shape[-1]
    out = np.empty((n, head_dim), dtype=np.float64)
    for i in range(n):
        _, off, pb, _ = slot_address(i, table_row, block_size)
        out[i] = upcast(_at(cache, pb, off, kv_head, layout), dtype)
    return out


def attention_weights(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Softmax over the scaled scores of one query against n keys.

    alpha_j = exp(q.K_j * scale) / sum_l exp(q.K_l * scale): the attention
    weights of §1.1 of the page "The KV Cache Problem of Traditional Attention"
    (pyllm.pages.dev) with scale = 1/sqrt(d_k), and the softmax of §1.2 of the
    page "Understanding KV Cache". The maximum score is subtracted before
    exponentiating; that leaves every ratio unchanged and keeps exp finite.
    """
    s = (K @ q) * scale
    e = np.exp(s - s.max())
    return e / e.sum()


def _attend_heads(qf: np.ndarray, gather_k, gather_v, num_kv_heads: int, n: int, scale: float) -> np.ndarray:
    """Query heads h of KV head h // g against that head's gathered K/V."""
    num_heads, head_dim = qf.shape
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = num_heads // num_kv_heads
    out = np.zeros((num_heads, head_dim), dtype=np.float64)
    if n == 0:
        return out
    for j in range(num_kv_heads):
        K, V = gather_k(j), gather_v(j)
        for h in range(j * group, (j + 1) * group):
            out[h] = attention_weights(qf[h], K, scale) @ V
    return out


def decode_attention_seq(q_b: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                         table_row: Sequence[int], n: int, scale: float, num_kv_heads: int,
                         block_size: int, dtype: str, layout: str = "HND") -> np.ndarray:
    """Output [num_heads, head_dim] (float64) of one sequence's decode step.

    Query head h reads KV head h // (num_heads / num_kv_heads): consecutive
    query heads share one KV head (page "KV Cache and Inference Optimization",
    section "Three attention layouts", GQA diagram). Decode at position n-1 is
    row n-1 of causal attention: the mask lets it see positions 0..n-1 (§1.2
    and §2.2 of the page "Understanding KV Cache"). n = 0 yields zeros.
    """
    return _attend_heads(upcast(q_b, dtype),
                         lambda j: gather_sequence(k_cache, dtype, table_row, n, j, block_size, layout),
                         lambda j: gather_sequence(v_cache, dtype, table_row, n, j, block_size, layout),
                         num_kv_heads, n, scale)


def decode_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     block_tables: np.ndarray, context_lens: Sequence[int], scale: float,
                     num_kv_heads: int, block_size: int, dtype: str,
                     seqs: Optional[Sequence[int]] = None, layout: str = "HND") -> np.ndarray:
    """Output [num_seqs, num_heads, head_dim] float64. With ``seqs`` only
    those sequences are computed and the other rows are NaN."""
    B, Hq, D = q.shape
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        out[b] = decode_attention_seq(q[b], k_cache, v_cache, block_tables[b], int(context_lens[b]),
                                      scale, num_kv_heads, block_size, dtype, layout)
    return out


def kv_append(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              slots: Sequence[int], block_size: int, layout: str = "HND") -> None:
    """Write each new token's K and V (all KV heads) into its slot, in place.

    The cache is an append-only log: each generated token adds one K/V record
    (§1.3 of the page "Understanding KV Cache"); slot s is offset s mod
    block_size of physical block s // block_size (§3.3). Slot -1 is skipped.
    Raw bytes are copied, so the write is exact.
    """
    for i, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        pb, off = s // block_size, s % block_size
        for j in range(k_new.shape[1]):
            _at(k_cache, pb, off, j, layout)[...] = k_new[i, j]
            _at(v_cache, pb, off, j, layout)[...] = v_new[i, j]


# ---------------------------------------------------------------------------
# FP8 (E4M3) caches: codes uint8 [NB, Hkv, bs, D], scales float32 [NB, Hkv, bs]
# (NHD: [NB, bs, Hkv, D] and [NB, bs, Hkv])
# ---------------------------------------------------------------------------
def gather_sequence_fp8(codes: np.ndarray, scales: np.ndarray, table_row: Sequence[int], n: int, kv_head: int,
                        block_size: int, layout: str = "HND", fmt: str = "e4m3") -> np.ndarray:
    """Contiguous float64 [n, D] of decode(code) * scale for one KV head
    (codes in format ``fmt``: "e4m3" or "int8")."""
    from .quant import decode_codes
    out = np.empty((n, codes.shape[-1]), dtype=np.float64)
    for i in range(n):
        _, off, pb, _ = slot_address(i, table_row, block_size)
        out[i] = decode_codes(_at(codes, pb, off, kv_head, layout), fmt) * np.float64(_at(scales, pb, off, kv_head,
                                                                                          layout))
    return out


def decode_attention_fp8(q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray,
                         v_scales: np.ndarray, block_tables: np.ndarray, context_lens: Sequence[int], scale: float,
                         num_kv_heads: int, block_size: int, q_dtype: str,
                         seqs: Optional[Sequence[int]] = None, layout: str = "HND",
                         fmt: str = "e4m3") -> np.ndarray:
    """Decode attention over 8-bit caches (FP8 E4M3 or INT8 codes): the same
    softmax attention, over the dequantized cached values."""
    B, Hq, D = q.shape
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        row = block_tables[b]
        out[b] = _attend_heads(upcast(q[b], q_dtype),
                               lambda j: gather_sequence_fp8(k_codes, k_scales, row, n, j, block_size, layout, fmt),
                               lambda j: gather_sequence_fp8(v_codes, v_scales, row, n, j, block_size, layout, fmt),
                               num_kv_heads, n, scale)
    return out


def kv_append_fp8(k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray, v_scales: np.ndarray,
                  k_new: np.ndarray, v_new: np.ndarray, slots: Sequence[int], block_size: int, in_dtype: str,
                  layout: str = "HND", fmt: str = "e4m3") -> None:
    """Quantize each new token's K and V rows (one scale per KV head row, see
    ``oracle.quant``; format ``fmt``) and write codes (raw bytes) and scales
    into the slot, in place."""
    from .quant import quantize_rows_fmt
    kq, ks = quantize_rows_fmt(upcast(k_new, in_dtype).astype(np.float32), fmt)
    vq, vs = quantize_rows_fmt(upcast(v_new, in_dtype).astype(np.float32), fmt)
    for i, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        pb, off = s // block_size, s % block_size
        for j in range(k_new.shape[1]):
            _at(k_codes, pb, off, j, layout)[...] = kq[i, j]
            _at(v_codes, pb, off, j, layout)[...] = vq[i, j]
            if layout == "HND":
                k_scales[pb, j, off] = ks[i, j]
                v_scales[pb, j, off] = vs[i, j]
            else:
                k_scales[pb, off, j] = ks[i, j]
                v_scales[pb, off, j] = vs[i, j]
