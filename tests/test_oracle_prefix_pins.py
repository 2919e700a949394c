"""Pins for the prefix-reuse and copy-on-write reference (``oracle/prefix.py``).

The pages state the rules in words ("KV Cache and Inference Optimization",
sections "PagedAttention" and "APC"): reuse walks a request's blocks from the
first, stops at the first miss, and reuses only whole blocks; shared blocks
are copied when a request diverges. The pins are hand-worked cases of those
rules, a closed form (longest common prefix), and planted mistakes.
"""
import itertools

import numpy as np
import pytest

from oracle import prefix as px


def test_hand_worked_reuse_rules():
    bs = 4
    cached = [[1, 2, 3, 4, 5, 6, 7, 8, 9, 10]]  # two full blocks + a partial one
    assert px.apc_hit_blocks(cached, [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12], bs) == 2  # partial block not reused
    assert px.apc_hit_blocks(cached, [1, 2, 3, 4, 5, 6, 0, 8], bs) == 1                  # diverges in block 1
    assert px.apc_hit_blocks(cached, [9, 9, 9, 9, 5, 6, 7, 8], bs) == 0                  # block 1 alike, block 0 not
    assert px.apc_hit_blocks(cached, [1, 2, 3], bs) == 0                                 # no full block
    assert px.apc_hit_blocks(cached, [1, 2, 3, 4], bs) == 1
    assert px.apc_hit_blocks([], [1, 2, 3, 4], bs) == 0
    # two cached requests: the walk may continue along either
    cached2 = cached + [[1, 2, 3, 4, 5, 6, 7, 0, 1, 1, 1, 1]]
    assert px.apc_hit_blocks(cached2, [1, 2, 3, 4, 5, 6, 7, 0, 1, 1, 1, 1, 2], bs) == 3
    assert px.apc_hit_blocks(cached2, [1, 2, 3, 4, 5, 6, 7, 8, 1, 1, 1, 1], bs) == 2
    # the same tokens at a different position are a different block
    assert px.apc_hit_blocks([[0, 0, 0, 0, 1, 2, 3, 4]], [1, 2, 3, 4], bs) == 0


def _lcp(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


@pytest.mark.parametrize("bs", [1, 2, 4, 16])
def test_closed_form_longest_common_prefix(bs):
    """hits = max over cached requests P of floor(lcp(P, R) / bs)."""
    rng = np.random.default_rng(bs)
    for _ in range(300):
        cached = [rng.integers(0, 3, rng.integers(0, 5 * bs + 3)).tolist() for _ in range(rng.integers(0, 4))]
        req = rng.integers(0, 3, rng.integers(0, 5 * bs + 3)).tolist()
        if cached and rng.random() < 0.5:  # force a long shared prefix
            base = cached[0]
            cut = int(rng.integers(0, len(base) + 1))
            req = base[:cut] + req
        want = max([_lcp(p, req) // bs for p in cached], default=0)
        assert px.apc_hit_blocks(cached, req, bs) == want


def test_exhaustive_tiny_alphabet():
    bs = 2
    seqs = [list(s) for n in range(0, 6) for s in itertools.product((0, 1), repeat=n)]
    cached = [[0, 1, 1, 0, 1], [1, 1, 0]]
    for r in seqs:
        assert px.apc_hit_blocks(cached, r, bs) == max(_lcp(p, r) // bs for p in cached)


def _no_stop_at_miss(cached, req, bs):
    """Planted mistake: count every block whose own tokens were cached at that position."""
    held = {(i, tuple(p[i * bs:(i + 1) * bs])) for p in cached for i in range(len(p) // bs)}
    return sum((i, tuple(req[i * bs:(i + 1) * bs])) in held for i in range(len(req) // bs))


def _partial_blocks_too(cached, req, bs):
    """Planted mistake: reuse the partial last block as well."""
    return max([_lcp(p, req) for p in cached], default=0) / bs


def test_planted_mistakes_fail_the_pins():
    bs = 4
    cached = [[1, 2, 3, 4, 5, 6, 7, 8, 9, 10]]
    req = [9, 9, 9, 9, 5, 6, 7, 8]
    assert _no_stop_at_miss(cached, req, bs) != px.apc_hit_blocks(cached, req, bs)
    req2 = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11]
    assert _partial_blocks_too(cached, req2, bs) != px.apc_hit_blocks(cached, req2, bs)


def test_copy_blocks_reference():
    cache = np.arange(6 * 3, dtype=np.float32).reshape(6, 3)
    before = cache.copy()
    px.copy_blocks(cache, [(0, 4), (2, 2), (7, 1), (1, -1), (3, 5)])
    want = before.copy()
    want[4] = before[0]
    want[5] = before[3]
    assert np.array_equal(cache, want)


def test_logical_sequences_fork_does_not_alias():
    ls = px.LogicalSequences()
    k = [np.full((2, 4), i, np.float32) for i in range(3)]
    ls.start(0, k, k)
    ls.fork(1, 0)
    ls.append(1, np.full((2, 4), 9, np.float32), np.full((2, 4), 9, np.float32))
    k0, _ = ls.kv(0)
    k1, _ = ls.kv(1)
    assert k0.shape == (3, 2, 4) and k1.shape == (4, 2, 4)
    assert np.array_equal(k1[:3], k0) and np.all(k1[3] == 9)
