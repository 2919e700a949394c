"""Seeded synthetic workloads for paged decode attention.

This module only draws random inputs and lays them out; it holds none of the
attention or slot arithmetic. Both the HIP path and the CPU reference consume
what it produces.

Shapes follow the model configurations printed on the page "The KV Cache
Problem of Traditional Attention" (pyllm.pages.dev, §1.2, ModelConfig table):
Llama-3-8B 32 query / 8 KV heads, Qwen2.5-7B 28 / 4, Llama-3-70B 64 / 8, all
with head_dim 128. The 16-token block is the default block size named on the
page "KV Cache and Inference Optimization" (note.yj-dis.top, section
"PagedAttention: manage the KV cache like virtual memory").

Recipe (every config):
  * seed = 156 + config index; numpy SeedSequence(seed).spawn(3) gives three
    independent streams: values, block permutation, context lengths;
  * values are i.i.d. N(0, 1) drawn in float32 and rounded once to the storage
    dtype with round-to-nearest-even;
  * the physical block pool holds exactly the blocks the sequences need plus
    one poison block, in an order given by a seeded permutation; every slot
    that is not part of a sequence's already-cached prefix holds NaN (the slot
    of the token about to be appended, the tail of each sequence's last block,
    the poison block), and block-table padding points at the poison block;
  * the large configurations draw their values on the GPU with torch's seeded
    generator (``fill_pool_device``) because tens of GiB of host-side draws
    would take minutes; the structure (lengths, permutation, tables) is always
    drawn on the host with numpy.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
BASE_SEED = 156


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One decode-attention workload (one layer's shape; ``num_layers`` pools)."""

    name: str
    index: int
    num_layers: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    context_lens: Optional[Sequence[int]] = None  # fixed lengths, or None
    context_len_range: Optional[tuple] = None  # (lo, hi) inclusive, uniform
    shared_prefix_tokens: int = 0
    pool_blocks: Optional[int] = None  # fixed pool size (tiny config)

    @property
    def group_size(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def scale(self) -> float:
        return float(self.head_dim) ** -0.5


CONFIGS = [
    DecodeConfig("tiny_fp32", 0, 1, 2, 4, 2, 64, 16, "f32",
                 context_lens=(18, 33), pool_blocks=16),
    DecodeConfig("llama3_8b_layer", 1, 32, 8, 32, 8, 128, 16, "bf16",
                 context_lens=(2048,) * 8),
    DecodeConfig("mha_contrast", 2, 32, 8, 32, 32, 128, 16, "bf16",
                 context_lens=(2048,) * 8),
    DecodeConfig("llama3_70b", 3, 80, 32, 64, 8, 128, 16, "bf16",
                 context_lens=(4096,) * 32),
    DecodeConfig("qwen25_7b_ragged", 4, 4, 64, 28, 4, 128, 16, "bf16",
                 context_len_range=(1, 32768), shared_prefix_tokens=512),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


def streams(seed: int):
    """Three independent generators: (values, permutation, lengths)."""
    ss = np.random.SeedSequence(seed)
    return tuple(np.random.default_rng(s) for s in ss.spawn(3))


# ---------------------------------------------------------------------------
# value drawing and storage rounding
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def storage_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(shape, 0x7FC0, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=storage_dtype(dtype))


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 rounded once to ``dtype`` storage (raw numpy array)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------------------------
# structure: lengths, block assignment, tables
# ---------------------------------------------------------------------------
def draw_context_lens(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.context_lens is not None:
        return np.asarray(cfg.context_lens, dtype=np.int32)
    lo, hi = cfg.context_len_range
    return rng.integers(lo, hi + 1, size=cfg.num_seqs, dtype=np.int64).astype(np.int32)


@dataclasses.dataclass
class BlockAssignment:
    """Physical block ids per sequence plus pool size and the poison block."""

    blocks: List[np.ndarray]  # per sequence, int32 physical ids, logical order
    num_blocks: int
    poison_block: int
    shared_ids: np.ndarray  # physical ids of the common prefix blocks, logical order
    shared_per_seq: List[int]  # how many leading logical blocks each sequence shares

    def table(self, max_blocks: Optional[int] = None, pad: Optional[int] = None) -> np.ndarray:
        """Dense int32 table ``[num_seqs, max_blocks]``; padding = ``pad``."""
        if max_blocks is None:
            max_blocks = max((len(b) for b in self.blocks), default=0)
        if pad is None:
            pad = self.poison_block
        t = np.full((len(self.blocks), max_blocks), pad, dtype=np.int32)
        for i, b in enumerate(self.blocks):
            t[i, : len(b)] = b
        return t


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def assign_blocks(context_lens: np.ndarray, block_size: int, rng: np.random.Generator,
                  shared_prefix_tokens: int = 0, pool_blocks: Optional[int] = None
                  ) -> BlockAssignment:
    """Seeded permutation of the pool over the sequences' logical blocks.

    With a shared prefix, logical blocks that lie wholly inside the prefix and
    strictly before the block that receives the sequence's newest token map to
    one common set of physical blocks; every other block is private.
    """
    n_shared_max = shared_prefix_tokens // block_size
    need = []
    shared_per_seq = []
    for n in context_lens:
        n = int(n)
        nb = ceil_div(n, block_size)
        last = (n - 1) // block_size if n > 0 else 0
        s = min(n_shared_max, last) if n > 0 else 0
        shared_per_seq.append(s)
        need.append(nb - s)
    common = n_shared_max if any(s > 0 for s in shared_per_seq) else 0
    total = common + sum(need) + 1  # + poison
    num_blocks = total if pool_blocks is None else pool_blocks
    if num_blocks < total:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {total}")
    perm = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    shared_ids = perm[cursor:cursor + common]
    cursor += common
    blocks = []
    for s, k in zip(shared_per_seq, need):
        own = perm[cursor:cursor + k]
        cursor += k
        blocks.append(np.concatenate([shared_ids[:s], own]).astype(np.int32))
    poison = int(perm[cursor])
    return BlockAssignment(blocks, num_blocks, poison, shared_ids.astype(np.int32), shared_per_seq)


@dataclasses.dataclass
class HostWorkload:
    """All inputs of one layer's decode step, as raw host arrays."""

    cfg: DecodeConfig
    context_lens: np.ndarray  # int32 [B]: tokens attended, incl. the new one
    assignment: BlockAssignment
    q: np.ndarray  # [B, Hq, D] raw storage
    k_new: np.ndarray  # [B, Hkv, D]
    v_new: np.ndarray
    k_cache: np.ndarray  # [num_blocks, Hkv, bs, D] raw storage, before append
    v_cache: np.ndarray

    @property
    def block_tables(self) -> np.ndarray:
        return self.assignment.table()


def make_host_workload(cfg: DecodeConfig, context_lens: Optional[Sequence[int]] = None,
                       seed: Optional[int] = None, pool_blocks: Optional[int] = None,
                       num_seqs: Optional[int] = None) -> HostWorkload:
    """Draw a full host-side workload (small shapes only: every value on CPU)."""
    seed = cfg.seed if seed is None else seed
    r_val, r_perm, r_len = streams(seed)
    if context_lens is None:
        lens = draw_context_lens(cfg, r_len)
    else:
        lens = np.asarray(context_lens, dtype=np.int32)
    if num_seqs is not None:
        lens = lens[:num_seqs]
    B, Hq, Hkv, D, bs = len(lens), cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    pool = cfg.pool_blocks if pool_blocks is None else pool_blocks
    asg = assign_blocks(lens, bs, r_perm, cfg.shared_prefix_tokens, pool)
    q = draw_values(r_val, (B, Hq, D), cfg.dtype)
    k_new = draw_values(r_val, (B, Hkv, D), cfg.dtype)
    v_new = draw_values(r_val, (B, Hkv, D), cfg.dtype)
    kc = nan_fill((asg.num_blocks, Hkv, bs, D), cfg.dtype)
    vc = nan_fill((asg.num_blocks, Hkv, bs, D), cfg.dtype)
    # The common prefix is drawn once per logical block; shared physical blocks
    # hold all of it, and a private block that replaces a shared one (the block
    # that receives a short sequence's newest token) starts as a copy of it.
    n_pref = len(asg.shared_ids)
    pk = [draw_values(r_val, (Hkv, bs, D), cfg.dtype) for _ in range(n_pref)]
    pv = [draw_values(r_val, (Hkv, bs, D), cfg.dtype) for _ in range(n_pref)]
    for lb, pb in enumerate(asg.shared_ids):
        kc[pb], vc[pb] = pk[lb], pv[lb]
    shared = set(int(x) for x in asg.shared_ids)
    # cached prefix of each sequence: positions [0, n-1); the slot of the new
    # token (position n-1) and everything after it stay NaN
    for b, n in enumerate(lens):
        n = int(n)
        for lb, pb in enumerate(asg.blocks[b]):
            pb = int(pb)
            if pb in shared:
                continue
            cnt = min(bs, max(0, n - 1 - lb * bs))
            if cnt <= 0:
                continue
            if lb < n_pref:
                kc[pb, :, :cnt], vc[pb, :, :cnt] = pk[lb][:, :cnt], pv[lb][:, :cnt]
            else:
                kc[pb, :, :cnt] = draw_values(r_val, (Hkv, cnt, D), cfg.dtype)
                vc[pb, :, :cnt] = draw_values(r_val, (Hkv, cnt, D), cfg.dtype)
    return HostWorkload(cfg, lens, asg, q, k_new, v_new, kc, vc)


def make_structure(cfg: DecodeConfig, seed: Optional[int] = None):
    """Lengths and block assignment only (for device-side value fills)."""
    seed = cfg.seed if seed is None else seed
    _, r_perm, r_len = streams(seed)
    lens = draw_context_lens(cfg, r_len)
    asg = assign_blocks(lens, cfg.block_size, r_perm, cfg.shared_prefix_tokens, cfg.pool_blocks)
    return lens, asg


# ---------------------------------------------------------------------------
# device-side fills (torch is imported lazily: the CPU tests never need it)
# ---------------------------------------------------------------------------
def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def fill_pool_device(t, generator):
    """Fill a device tensor with N(0,1) in float32, rounded to its dtype."""
    import torch
    flat = t.view(-1)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        tmp = torch.randn(e - s, generator=generator, device=t.device, dtype=torch.float32)
        flat[s:e].copy_(tmp)
    return t


def poison_device_pool(k_cache, v_cache, context_lens, assignment: BlockAssignment, block_size: int):
    """Copy-on-write set-up of private prefix blocks, then NaN into the poison
    block and into every slot at or after each sequence's position n-1."""
    nan = float("nan")
    n_pref = len(assignment.shared_ids)
    shared = set(int(x) for x in assignment.shared_ids)
    for b, blocks in enumerate(assignment.blocks):
        for lb in range(min(n_pref, len(blocks))):
            pb = int(blocks[lb])
            if pb not in shared:
                src = int(assignment.shared_ids[lb])
                k_cache[pb].copy_(k_cache[src])
                v_cache[pb].copy_(v_cache[src])
    k_cache[assignment.poison_block].fill_(nan)
    v_cache[assignment.poison_block].fill_(nan)
    for b, n in enumerate(context_lens):
        n = int(n)
        if n == 0:
            continue
        lb = (n - 1) // block_size
        off = (n - 1) % block_size
        pb = int(assignment.blocks[b][lb])
        k_cache[pb, :, off:, :].fill_(nan)
        v_cache[pb, :, off:, :].fill_(nan)
    return k_cache, v_cache


# ---------------------------------------------------------------------------
# raw host arrays <-> torch device tensors (bit-preserving)
# ---------------------------------------------------------------------------
def raw_to_torch(raw: np.ndarray, dtype: str, device):
    import torch
    raw = np.ascontiguousarray(raw)
    if dtype == "bf16":
        t = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(raw)
    return t.to(device)


def torch_to_raw(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@dataclasses.dataclass
class DeviceWorkload:
    """One decode step's inputs resident in device memory, for ``layers``
    layers that share one block table (each layer has its own K/V pools)."""

    cfg: DecodeConfig
    context_lens: np.ndarray
    assignment: BlockAssignment
    q: list  # per layer [B, Hq, D]
    k_new: list
    v_new: list
    k_cache: list  # per layer [NB, Hkv, bs, D]
    v_cache: list
    block_tables: object  # device int32 [B, maxNB]
    context_lens_dev: object  # device int32 [B]

    @property
    def layers(self) -> int:
        return len(self.k_cache)


def value_generator(seed: int, device):
    import torch
    g = torch.Generator(device=device)
    # the values stream of the config's seed, reduced to a torch seed
    g.manual_seed(int(streams(seed)[0].integers(0, 2 ** 62)))
    return g


def make_device_workload(cfg: DecodeConfig, device, layers: int = 1, seed: Optional[int] = None,
                         context_lens: Optional[np.ndarray] = None,
                         assignment: Optional[BlockAssignment] = None, progress=None) -> DeviceWorkload:
    """Structure on the host (numpy) unless given, values drawn on the device
    (torch). ``assignment`` lets a caller supply block lists built elsewhere
    (e.g. by a block allocator) for ``context_lens``."""
    import torch
    seed = cfg.seed if seed is None else seed
    if assignment is None:
        lens, asg = make_structure(cfg, seed)
    else:
        lens, asg = np.asarray(context_lens, np.int32), assignment
    gen = value_generator(seed, device)
    tdt = torch_dtype(cfg.dtype)
    B, Hq, Hkv, D, bs = len(lens), cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    qs, kns, vns, kcs, vcs = [], [], [], [], []
    for _ in range(layers):
        kc = fill_pool_device(torch.empty((asg.num_blocks, Hkv, bs, D), dtype=tdt, device=device), gen)
        vc = fill_pool_device(torch.empty((asg.num_blocks, Hkv, bs, D), dtype=tdt, device=device), gen)
        poison_device_pool(kc, vc, lens, asg, bs)
        kcs.append(kc)
        vcs.append(vc)
        qs.append(fill_pool_device(torch.empty((B, Hq, D), dtype=tdt, device=device), gen))
        kns.append(fill_pool_device(torch.empty((B, Hkv, D), dtype=tdt, device=device), gen))
        vns.append(fill_pool_device(torch.empty((B, Hkv, D), dtype=tdt, device=device), gen))
        if progress is not None:
            progress(len(kcs))
    tables = torch.from_numpy(asg.table()).to(device)
    lens_dev = torch.from_numpy(lens.astype(np.int32)).to(device)
    return DeviceWorkload(cfg, lens, asg, qs, kns, vns, kcs, vcs, tables, lens_dev)


# ---------------------------------------------------------------------------
# FP8 (E4M3) caches: the cached codes and per-row scales are drawn directly as
# input data (any finite code, scales spread over an order of magnitude); the
# new tokens' K/V are drawn like every other value and quantized by the path.
# ---------------------------------------------------------------------------
FP8_NAN = 0x7F


def draw_fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ np.uint8(1), c).astype(np.uint8)  # no NaN codes


def draw_fp8_scales(rng: np.random.Generator, shape) -> np.ndarray:
    return (rng.uniform(0.3, 3.0, size=shape) / 448.0).astype(np.float32)


@dataclasses.dataclass
class HostWorkloadFp8:
    cfg: DecodeConfig  # cfg.dtype is the query / output / new-token type
    context_lens: np.ndarray
    assignment: BlockAssignment
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    k_codes: np.ndarray  # uint8 [NB, Hkv, bs, D]
    v_codes: np.ndarray
    k_scales: np.ndarray  # float32 [NB, Hkv, bs]
    v_scales: np.ndarray

    @property
    def block_tables(self) -> np.ndarray:
        return self.assignment.table()


def make_host_workload_fp8(cfg: DecodeConfig, context_lens: Optional[Sequence[int]] = None,
                           seed: Optional[int] = None, pool_blocks: Optional[int] = None) -> HostWorkloadFp8:
    seed = cfg.seed if seed is None else seed
    r_val, r_perm, r_len = streams(seed)
    lens = draw_context_lens(cfg, r_len) if context_lens is None else np.asarray(context_lens, dtype=np.int32)
    B, Hq, Hkv, D, bs = len(lens), cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    pool = cfg.pool_blocks if pool_blocks is None else pool_blocks
    asg = assign_blocks(lens, bs, r_perm, cfg.shared_prefix_tokens, pool)
    q = draw_values(r_val, (B, Hq, D), cfg.dtype)
    k_new = draw_values(r_val, (B, Hkv, D), cfg.dtype)
    v_new = draw_values(r_val, (B, Hkv, D), cfg.dtype)
    kc = np.full((asg.num_blocks, Hkv, bs, D), FP8_NAN, np.uint8)
    vc = np.full((asg.num_blocks, Hkv, bs, D), FP8_NAN, np.uint8)
    ks = np.full((asg.num_blocks, Hkv, bs), np.nan, np.float32)
    vs = np.full((asg.num_blocks, Hkv, bs), np.nan, np.float32)
    n_pref = len(asg.shared_ids)
    pref = [(draw_fp8_codes(r_val, (Hkv, bs, D)), draw_fp8_codes(r_val, (Hkv, bs, D)),
             draw_fp8_scales(r_val, (Hkv, bs)), draw_fp8_scales(r_val, (Hkv, bs))) for _ in range(n_pref)]
    for lb, pb in enumerate(asg.shared_ids):
        kc[pb], vc[pb], ks[pb], vs[pb] = pref[lb]
    shared = set(int(x) for x in asg.shared_ids)
    for b, n in enumerate(lens):
        n = int(n)
        for lb, pb in enumerate(asg.blocks[b]):
            pb = int(pb)
            if pb in shared:
                continue
            cnt = min(bs, max(0, n - 1 - lb * bs))
            if cnt <= 0:
                continue
            if lb < n_pref:
                src = pref[lb]
                kc[pb, :, :cnt], vc[pb, :, :cnt] = src[0][:, :cnt], src[1][:, :cnt]
                ks[pb, :, :cnt], vs[pb, :, :cnt] = src[2][:, :cnt], src[3][:, :cnt]
            else:
                kc[pb, :, :cnt] = draw_fp8_codes(r_val, (Hkv, cnt, D))
                vc[pb, :, :cnt] = draw_fp8_codes(r_val, (Hkv, cnt, D))
                ks[pb, :, :cnt] = draw_fp8_scales(r_val, (Hkv, cnt))
                vs[pb, :, :cnt] = draw_fp8_scales(r_val, (Hkv, cnt))
    return HostWorkloadFp8(cfg, lens, asg, q, k_new, v_new, kc, vc, ks, vs)


@dataclasses.dataclass
class DeviceWorkloadFp8:
    cfg: DecodeConfig
    context_lens: np.ndarray
    assignment: BlockAssignment
    q: list
    k_new: list
    v_new: list
    k_codes: list  # per layer uint8 [NB, Hkv, bs, D]
    v_codes: list
    k_scales: list  # per layer float32 [NB, Hkv, bs]
    v_scales: list
    block_tables: object
    context_lens_dev: object

    @property
    def layers(self) -> int:
        return len(self.k_codes)


def fill_codes_device(t, generator):
    import torch
    flat = t.view(-1)
    chunk = 1 << 28
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        c = torch.randint(0, 256, (e - s,), generator=generator, device=t.device, dtype=torch.int32)
        c = torch.where((c & 0x7F) == 0x7F, c ^ 1, c)
        flat[s:e].copy_(c)
    return t


def make_device_workload_fp8(cfg: DecodeConfig, device, layers: int = 1, seed: Optional[int] = None,
                             context_lens: Optional[np.ndarray] = None,
                             assignment: Optional[BlockAssignment] = None) -> DeviceWorkloadFp8:
    import torch
    seed = cfg.seed if seed is None else seed
    if assignment is None:
        lens, asg = make_structure(cfg, seed)
    else:
        lens, asg = np.asarray(context_lens, np.int32), assignment
    gen = value_generator(seed, device)
    tdt = torch_dtype(cfg.dtype)
    B, Hq, Hkv, D, bs = len(lens), cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    out = dict(q=[], k_new=[], v_new=[], k_codes=[], v_codes=[], k_scales=[], v_scales=[])
    for _ in range(layers):
        for name in ("k_codes", "v_codes"):
            out[name].append(fill_codes_device(torch.empty((asg.num_blocks, Hkv, bs, D), dtype=torch.uint8,
                                                           device=device), gen))
        for name in ("k_scales", "v_scales"):
            sc = torch.rand((asg.num_blocks, Hkv, bs), generator=gen, device=device, dtype=torch.float32)
            out[name].append(sc.mul_(2.7).add_(0.3).div_(448.0))
        # copy-on-write set-up and poison, as for 16-bit caches
        n_pref = len(asg.shared_ids)
        shared = set(int(x) for x in asg.shared_ids)
        for b, blocks in enumerate(asg.blocks):
            for lb in range(min(n_pref, len(blocks))):
                pb = int(blocks[lb])
                if pb not in shared:
                    src = int(asg.shared_ids[lb])
                    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
                        out[name][-1][pb].copy_(out[name][-1][src])
        for name in ("k_codes", "v_codes"):
            out[name][-1][asg.poison_block].fill_(FP8_NAN)
        for name in ("k_scales", "v_scales"):
            out[name][-1][asg.poison_block].fill_(float("nan"))
        for b, n in enumerate(lens):
            n = int(n)
            if n == 0:
                continue
            pb = int(asg.blocks[b][(n - 1) // bs])
            off = (n - 1) % bs
            for name in ("k_codes", "v_codes"):
                out[name][-1][pb, :, off:].fill_(FP8_NAN)
            for name in ("k_scales", "v_scales"):
                out[name][-1][pb, :, off:].fill_(float("nan"))
        for name, shape in (("q", (B, Hq, D)), ("k_new", (B, Hkv, D)), ("v_new", (B, Hkv, D))):
            out[name].append(fill_pool_device(torch.empty(shape, dtype=tdt, device=device), gen))
    tables = torch.from_numpy(asg.table()).to(device)
    lens_dev = torch.from_numpy(lens.astype(np.int32)).to(device)
    return DeviceWorkloadFp8(cfg, lens, asg, out["q"], out["k_new"], out["v_new"], out["k_codes"], out["v_codes"],
                             out["k_scales"], out["v_scales"], tables, lens_dev)


def to_layout(cache: np.ndarray, layout: str) -> np.ndarray:
    """A [NB, Hkv, bs, ...] host cache (HND) in ``layout``: unchanged for "HND",
    axes 1 and 2 swapped (a contiguous copy) for "NHD" = [NB, bs, Hkv, ...]."""
    if layout == "HND":
        return cache
    if layout == "NHD":
        return np.ascontiguousarray(np.swapaxes(cache, 1, 2))
    raise ValueError(f"unknown layout {layout!r}")
