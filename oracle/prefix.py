"""Prefix reuse and copy-on-write, as plain Python / NumPy.

Test infrastructure only (see the package docstring).

Page "KV Cache and Inference Optimization", sections "PagedAttention" and
"APC":
  * blocks with the same prefix are stored once and referenced by several
    requests; a request that diverges inside a shared block gets its own copy
    (copy-on-write);
  * a request reuses cached blocks from its first block on, block by block,
    and stops at the first block that is not cached: after one miss no later
    block can be reused; only whole blocks are reused.
Page "Why does a request use more memory the longer it generates?", section
"Paging changes allocation, not a token's representation": reused state must
match the exact token sequence and positions (and the model).

Reading used here: a block of a new request is "cached" when some earlier
request registered a block holding the same tokens at the same positions
after the same preceding tokens, i.e. the registered token sequence and the
request agree on every token up to the end of that block. That is the
content of a prefix, compared exactly; no hashing is involved.
"""
from __future__ import annotations

from typing import Iterable, List, Sequence

import numpy as np


def cached_full_blocks(registered: Iterable[Sequence[int]], block_size: int) -> set:
    """Every prefix (as a tuple of tokens) that ends at a full-block boundary
    of some registered token sequence: the content the cache holds."""
    held = set()
    for toks in registered:
        toks = tuple(int(t) for t in toks)
        for i in range(len(toks) // block_size):
            held.add(toks[: (i + 1) * block_size])
    return held


def apc_hit_blocks(registered: Iterable[Sequence[int]], request: Sequence[int], block_size: int) -> int:
    """Leading full blocks of `request` found in the cache, walking from the
    first block and stopping at the first miss."""
    held = cached_full_blocks(registered, block_size)
    req = tuple(int(t) for t in request)
    hits = 0
    for i in range(len(req) // block_size):
        if req[: (i + 1) * block_size] in held:
            hits += 1
        else:
            break
    return hits


def copy_blocks(cache: np.ndarray, pairs: Sequence[Sequence[int]]) -> None:
    """cache[dst] = cache[src] for each (src, dst), in place; pairs with an
    id outside the cache or src == dst are skipped."""
    nb = cache.shape[0]
    for src, dst in pairs:
        if src == dst or not (0 <= src < nb) or not (0 <= dst < nb):
            continue
        cache[dst] = cache[src]


class LogicalSequences:
    """What every sequence holds, independent of where its blocks live: a
    list of (K, V) rows per sequence, in position order. Forking copies the
    list; appending adds one row. Paging, sharing and copy-on-write change
    only where rows are stored, never these lists."""

    def __init__(self):
        self.rows: dict = {}

    def start(self, seq: int, k_rows: Sequence[np.ndarray], v_rows: Sequence[np.ndarray]) -> None:
        self.rows[seq] = [(np.array(k), np.array(v)) for k, v in zip(k_rows, v_rows)]

    def fork(self, dst: int, src: int) -> None:
        self.rows[dst] = list(self.rows[src])

    def append(self, seq: int, k: np.ndarray, v: np.ndarray) -> None:
        self.rows[seq].append((np.array(k), np.array(v)))

    def kv(self, seq: int):
        """(K [n, Hkv, D], V [n, Hkv, D]) of one sequence."""
        r: List = self.rows[seq]
        return np.stack([k for k, _ in r]), np.stack([v for _, v in r])
