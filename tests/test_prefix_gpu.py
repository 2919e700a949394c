"""GPU tests of prefix sharing: the copy-on-write block copy (bit-exact
against the reference copy), and whole decode runs over forked and
prefix-cached sequences, checked against the reference attention over each
sequence's logical rows (what the sequence holds, wherever its blocks live).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from paged_kv_cache_156_amd import binding as pkv
from paged_kv_cache_156_amd import workloads as wl

pytestmark = pytest.mark.gpu
BS = 16


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load()
    return torch, torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(got, ref, what, dtype="bf16"):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = (1e-5 + 1e-5 * np.abs(ref)) if dtype == "f32" else (2e-3 + 1e-2 * np.abs(ref))
    assert (err <= bound).all(), f"{what}: max|err|={err.max():.3e}"


@pytest.mark.parametrize("kind", ["bf16", "f32", "fp8"])
def test_copy_blocks_bit_exact(torch_dev, kind):
    torch, dev = torch_dev
    note(f"copy_blocks {kind}")
    rng = np.random.default_rng(11)
    NB, Hkv, D = 40, 4, 128
    if kind == "fp8":
        host = [rng.integers(0, 256, (NB, Hkv, BS, D), dtype=np.uint8), rng.integers(0, 256, (NB, Hkv, BS, D),
                dtype=np.uint8), rng.standard_normal((NB, Hkv, BS)).astype(np.float32),
                rng.standard_normal((NB, Hkv, BS)).astype(np.float32)]
    else:
        host = [wl.draw_values(rng, (NB, Hkv, BS, D), kind) for _ in range(2)]
    dev_t = [torch.from_numpy(h.copy()).to(dev) for h in host]
    pairs = np.array([[0, 5], [7, 30], [3, 3], [39, 1], [2, 45], [-1, 6], [12, 13], [14, 20]], np.int32)
    pkv.copy_blocks(dev_t, torch.from_numpy(pairs).to(dev))
    torch.cuda.synchronize()
    for h, d in zip(host, dev_t):
        want = h.copy()
        oracle.copy_blocks(want, pairs.tolist())
        assert d.cpu().numpy().tobytes() == want.tobytes()
    # no pairs: a no-op
    pkv.copy_blocks(dev_t, torch.zeros((0, 2), dtype=torch.int32, device=dev))


def logical_attention(q_b, k_rows, v_rows, scale, Hkv, dtype):
    """Reference decode output of one sequence from its logical rows [n, Hkv, D]."""
    n, _, D = k_rows.shape
    nblk = -(-n // BS)
    kc = wl.nan_fill((nblk, Hkv, BS, D), dtype)
    vc = wl.nan_fill((nblk, Hkv, BS, D), dtype)
    for t in range(n):
        kc[t // BS, :, t % BS] = k_rows[t]
        vc[t // BS, :, t % BS] = v_rows[t]
    return oracle.decode_attention_seq(q_b, kc, vc, list(range(nblk)), n, scale, Hkv, BS, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forked_sequences_decode_with_copy_on_write(torch_dev, dtype):
    """Beam-style forks: one prefill, forks that share it (partial block
    included), then decode steps where every sequence appends its own token.
    Each step: pool appends (copy pairs) -> copy_blocks -> decode (fused step
    on even steps, append + split attention on odd ones); every output is
    compared with the reference over the sequence's logical rows, and at the
    end every sequence read back through its block table must equal its rows
    bit for bit."""
    torch, dev = torch_dev
    rng = np.random.default_rng(21)
    Hq, Hkv, D = 8, 2, 128
    scale = D ** -0.5
    NB, MAXB = 64, 8
    pool = pkv.BlockPool(NB, BS, max_seqs=8, seed=5)
    kc = wl.raw_to_torch(wl.nan_fill((NB, Hkv, BS, D), dtype), dtype, dev)
    vc = wl.raw_to_torch(wl.nan_fill((NB, Hkv, BS, D), dtype), dtype, dev)
    logical = oracle.LogicalSequences()
    n0 = 37
    k0, v0 = wl.draw_values(rng, (n0, Hkv, D), dtype), wl.draw_values(rng, (n0, Hkv, D), dtype)
    pool.grow(0, n0)
    slots = pool.slot_mapping([0] * n0, range(n0))
    pkv.kv_append(wl.raw_to_torch(k0, dtype, dev), wl.raw_to_torch(v0, dtype, dev), torch.from_numpy(slots).to(dev),
                  kc, vc)
    logical.start(0, list(k0), list(v0))
    for s in (1, 2):
        pool.fork(s, 0)
        logical.fork(s, 0)
    seqs = [0, 1, 2]
    copies = 0
    for step in range(24):
        if step == 5:
            pool.fork(3, 1)
            logical.fork(3, 1)
            seqs = [0, 1, 2, 3]
        if step == 11:
            pool.free(2)
            del logical.rows[2]
            seqs = [0, 1, 3]
        note(f"fork/CoW {dtype} step {step}: seqs {seqs}")
        slots, pairs = pool.append_slots(seqs)
        copies += len(pairs)
        pkv.copy_blocks([kc, vc], torch.from_numpy(pairs.astype(np.int32)).to(dev))
        B = len(seqs)
        q = wl.draw_values(rng, (B, Hq, D), dtype)
        kn, vn = wl.draw_values(rng, (B, Hkv, D), dtype), wl.draw_values(rng, (B, Hkv, D), dtype)
        for i, s in enumerate(seqs):
            logical.append(s, kn[i], vn[i])
        lens = np.array([pool.seq_info(s)[0] for s in seqs], np.int32)
        table = pool.block_tables(seqs, MAXB)
        qd, knd, vnd = (wl.raw_to_torch(x, dtype, dev) for x in (q, kn, vn))
        td, ld = torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev)
        out = torch.full_like(qd, float("nan"))
        if step % 2 == 0:
            ws = pkv.alloc_step_workspace(qd, kc, td, 1)
            pkv.decode_step(qd, knd, vnd, kc, vc, td, ld, scale, out, ws, 1)
        else:
            pkv.kv_append(knd, vnd, torch.from_numpy(slots).to(dev), kc, vc)
            ws = pkv.alloc_workspace(qd, kc, td, 1)
            pkv.paged_decode_attention(qd, kc, vc, td, ld, scale, out, ws, 1)
        torch.cuda.synchronize()
        got = oracle.upcast(wl.torch_to_raw(out, dtype), dtype)
        for i, s in enumerate(seqs):
            kr, vr = logical.kv(s)
            ref = logical_attention(q[i], kr, vr, scale, Hkv, dtype)
            check_close(got[i], ref, f"step {step} seq {s}", dtype)
    assert copies >= 3  # the forks really diverged inside shared blocks
    kh, vh = wl.torch_to_raw(kc, dtype), wl.torch_to_raw(vc, dtype)
    for s in seqs:
        n, blocks = pool.seq_info(s)
        kr, vr = logical.kv(s)
        for j in range(Hkv):
            assert np.array_equal(oracle.gather_sequence(kh, dtype, blocks, n, j, BS), oracle.upcast(kr[:, j], dtype))
            assert np.array_equal(oracle.gather_sequence(vh, dtype, blocks, n, j, BS), oracle.upcast(vr[:, j], dtype))


def rows_for_prefix(tokens, Hkv, D, dtype):
    """K/V rows of each position as a function of the exact token prefix that
    ends there (a stand-in for a model: same prefix -> same state)."""
    ks, vs = [], []
    for p in range(len(tokens)):
        seed = zlib.crc32(np.asarray(tokens[: p + 1], np.int64).tobytes())
        r = np.random.default_rng(seed)
        ks.append(wl.draw_values(r, (Hkv, D), dtype))
        vs.append(wl.draw_values(r, (Hkv, D), dtype))
    return np.stack(ks), np.stack(vs)


def test_prefix_cache_reuse_decode(torch_dev):
    """Requests sharing a system prompt reuse its cached full blocks and
    compute K/V only after the hit; the decode over the reused blocks must
    equal the reference over the request's own rows."""
    torch, dev = torch_dev
    dtype, Hq, Hkv, D = "bf16", 8, 2, 128
    scale = D ** -0.5
    NB, MAXB = 64, 8
    rng = np.random.default_rng(33)
    pool = pkv.BlockPool(NB, BS, max_seqs=8, seed=9)
    kc = wl.raw_to_torch(wl.nan_fill((NB, Hkv, BS, D), dtype), dtype, dev)
    vc = wl.raw_to_torch(wl.nan_fill((NB, Hkv, BS, D), dtype), dtype, dev)
    system = rng.integers(0, 1000, 40).tolist()
    prompts = [system + rng.integers(0, 1000, 10).tolist(),
               system + rng.integers(0, 1000, 15).tolist(),
               system[:20] + rng.integers(0, 1000, 30).tolist(),
               rng.integers(0, 1000, 33).tolist()]
    want_hits = [0, 32, 16, 0]
    registered = []
    for s, toks in enumerate(prompts):
        hit = pool.adopt_prefix(s, toks)
        assert hit == want_hits[s] == BS * oracle.apc_hit_blocks(registered, toks, BS)
        pool.grow(s, len(toks))
        kr, vr = rows_for_prefix(toks, Hkv, D, dtype)
        pos = np.arange(hit, len(toks))
        slots = pool.slot_mapping([s] * len(pos), pos)  # only the blocks after the hit: never shared
        pkv.kv_append(wl.raw_to_torch(kr[hit:], dtype, dev), wl.raw_to_torch(vr[hit:], dtype, dev),
                      torch.from_numpy(slots).to(dev), kc, vc)
        pool.prefix_register(s, toks)
        registered.append(toks)
    note(f"prefix cache: hits {want_hits}, stats {pool.prefix_stats()}")
    seqs = list(range(len(prompts)))
    for step in range(3):
        for s in seqs:
            prompts[s] = prompts[s] + [int(rng.integers(0, 1000))]
        slots, pairs = pool.append_slots(seqs)
        assert len(pairs) == 0  # cached blocks are full: appends never land in them
        rows = [rows_for_prefix(prompts[s], Hkv, D, dtype) for s in seqs]
        kn = np.stack([r[0][-1] for r in rows])
        vn = np.stack([r[1][-1] for r in rows])
        q = wl.draw_values(rng, (len(seqs), Hq, D), dtype)
        lens = np.array([len(prompts[s]) for s in seqs], np.int32)
        assert lens.tolist() == [pool.seq_info(s)[0] for s in seqs]
        td = torch.from_numpy(pool.block_tables(seqs, MAXB)).to(dev)
        qd = wl.raw_to_torch(q, dtype, dev)
        out = torch.full_like(qd, float("nan"))
        ws = pkv.alloc_step_workspace(qd, kc, td, 2)
        pkv.decode_step(qd, wl.raw_to_torch(kn, dtype, dev), wl.raw_to_torch(vn, dtype, dev), kc, vc, td,
                        torch.from_numpy(lens).to(dev), scale, out, ws, 2)
        torch.cuda.synchronize()
        got = oracle.upcast(wl.torch_to_raw(out, dtype), dtype)
        for i, s in enumerate(seqs):
            ref = logical_attention(q[i], rows[i][0], rows[i][1], scale, Hkv, dtype)
            check_close(got[i], ref, f"prefix reuse step {step} seq {s}")
