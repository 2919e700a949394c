#!/usr/bin/env python3
"""Decode-step benchmark of libpkv on one MI355X.

One step = for every layer: append the new token's K/V, then paged decode
attention over the whole cache. Default (--mode fused): one pkv_decode_step
launch per layer (append + attention + merge); --mode split: kv_append,
decode_partitions and decode_merge as three launches.
Default workload: Llama-3-70B shape (64 query / 8 KV heads, head_dim 128,
bf16), batch 32, context 4096, 80 layers looped, each layer with its own
K/V pool (40 GiB resident) and one block table shared by the layers, built
by libpkv's block pool from a seeded permutation.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--layers L]
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth, decimal GB/s
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_156_amd", "csrc", "pkv_kernels.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def copy_calibration(args, torch, dev):
    """--copy-calibration-mib: one device-to-device copy of that size, so a
    counter run can read FETCH_SIZE / WRITE_SIZE for known bytes beside the
    kernel it measures."""
    if not args.copy_calibration_mib:
        return
    n = args.copy_calibration_mib * 2**20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {args.copy_calibration_mib} MiB device-to-device copy done")


def settle(fn, torch, settle_ms):
    """Repeat `fn` untimed until the GPU has run it for `settle_ms` (batches of
    about 5 ms, host clock around each synchronised batch); returns the count.
    Launches start below their sustained rate: the 70B prefill launch (MFMA
    bound) measured ~25% slower over its first ~60 ms of back-to-back work
    than afterwards; the 70B 8-bit decode launch ran at its final rate for
    about 2 ms, then 10-20% slower (INT8) or 2-5% slower (E4M3) until about
    15 ms in (16-bit: within 1% throughout)."""
    if settle_ms <= 0:
        return 0
    torch.cuda.synchronize()
    t = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t, 1e-6)
    batch = max(1, int(5e-3 / one))
    n, t0 = 1, time.perf_counter()
    while (time.perf_counter() - t0 + one) * 1e3 < settle_ms:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        n += batch
    return n


def profile_traffic(name, pb):
    """HBM bytes per launch from a committed counter summary under profiles/,
    if it was taken on this kernel source and partition size (else None)."""
    tfile = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(tfile):
        return None
    with open(tfile) as f:
        tr = json.load(f)
    if tr.get("kernel_sha") == kernel_sha() and tr.get("partition_blocks") == pb:
        return tr.get("bytes_per_launch")
    return None


def pool_assignment(cfg, lens, pkv, wl):
    """Block lists, slot mapping and tables from libpkv's host block pool."""
    bs = cfg.block_size
    B = len(lens)
    n_pref = cfg.shared_prefix_tokens // bs
    share = [min(n_pref, (int(n) - 1) // bs) if (n_pref and n > 0) else 0 for n in lens]
    need = (n_pref if any(share) else 0) + sum(-(-int(n) // bs) - s for n, s in zip(lens, share))
    pool = pkv.BlockPool(max(need, 1), bs, max_seqs=B + 1, seed=cfg.seed)
    owner = B  # bookkeeping sequence that holds the shared prefix blocks
    if any(share):
        pool.grow(owner, n_pref * bs)
    for b, n in enumerate(lens):
        if share[b]:
            pool.share_prefix(b, owner, share[b] * bs)
        pool.grow(b, int(n))
    blocks = [pool.seq_info(b)[1] for b in range(B)]
    shared_ids = pool.seq_info(owner)[1] if any(share) else np.zeros(0, np.int32)
    poison = max(need, 1)  # one extra block past the pool: NaN, target of table padding
    slots = pool.slot_mapping(np.arange(B), np.asarray(lens) - 1)
    asg = wl.BlockAssignment(blocks, poison + 1, poison, shared_ids.astype(np.int32), share)
    return asg, slots, pool.stats()


def snapshot_layer0(wkd, fp8, dt):
    """Host copies of layer 0's inputs, taken before any step runs: the whole
    K/V pools in the timed layout (the new token's slot still holds NaN), the
    queries, the new K/V rows, the block tables and the lengths."""
    if fp8:
        pools = [wkd.k_codes[0].cpu().numpy(), wkd.v_codes[0].cpu().numpy(), wkd.k_scales[0].cpu().numpy(),
                 wkd.v_scales[0].cpu().numpy()]
    else:
        pools = [wl_raw(wkd.k_cache[0], dt), wl_raw(wkd.v_cache[0], dt)]
    return dict(pools=pools, q=wl_raw(wkd.q[0], dt), kn=wl_raw(wkd.k_new[0], dt), vn=wl_raw(wkd.v_new[0], dt),
                table=wkd.block_tables.cpu().numpy(), lens=np.asarray(wkd.context_lens, np.int32).copy())


def wl_raw(t, dt):
    from paged_kv_cache_156_amd import workloads as wl
    return wl.torch_to_raw(t, dt)


def pools_after(wkd, fp8, dt):
    """Host copies of layer 0's pools as the timed steps left them."""
    if fp8:
        return [wkd.k_codes[0].cpu().numpy(), wkd.v_codes[0].cpu().numpy(), wkd.k_scales[0].cpu().numpy(),
                wkd.v_scales[0].cpu().numpy()]
    return [wl_raw(wkd.k_cache[0], dt), wl_raw(wkd.v_cache[0], dt)]


def decode_alg_bytes(lens, Hq, Hkv, D, esz, bs, fp8, fused):
    """Algorithmic bytes of one decode launch over one layer, as
    (K/V bytes, launch bytes): every cached K/V row read once (8-bit caches:
    the codes plus one fp32 scale per row), the queries read and the outputs
    written, the block-table entries each sequence reads plus its length, and
    for the fused step the new token's K/V read and its row written."""
    B = len(lens)
    sum_n = int(sum(int(n) for n in lens))
    kv_layer = 2 * Hkv * (D + 4) * sum_n if fp8 else 2 * Hkv * D * esz * sum_n
    q_out = 2 * B * Hq * D * esz
    tables = 4 * sum(-(-int(n) // bs) for n in lens) + 4 * B
    append = 2 * B * Hkv * D * esz + (2 * B * Hkv * (D + 4) if fp8 else 2 * B * Hkv * D * esz)
    return kv_layer, kv_layer + q_out + tables + (append if fused else 0)


def oracle_check(snap, out0, after, cfg, layout, fp8, fmt, budget_s, min_seqs=32):
    """The CPU reference on layer 0, timed, and compared with the GPU.

    The reference appends every sequence's new token at its slot in the whole
    layer-0 pool (the slot rule applied to the same block tables the GPU used),
    then attends sequence by sequence through those tables until ``budget_s``
    of work is done and at least ``min_seqs`` sequences (or all of them) are
    checked. Each checked sequence's output is compared element by element with
    the timed run's layer-0 output; the appended pools are compared byte for
    byte with the GPU's. Runs on one thread: the reference gathers token by
    token in a Python loop, whatever BLAS could offer.
    """
    import oracle
    from threadpoolctl import threadpool_limits
    dt, bs, Hkv = cfg.dtype, cfg.block_size, cfg.num_kv_heads
    table, lens = snap["table"], snap["lens"]
    pools = [p.copy() for p in snap["pools"]]
    B = len(lens)
    atol, rtol = (1e-5, 1e-5) if dt == "f32" else (2e-3, 1e-2)
    esz = 1 if fp8 else (4 if dt == "f32" else 2)
    row_bytes = cfg.head_dim * esz + (4 if fp8 else 0)
    done, kv_bytes, worst, worst_ratio, bad = 0, 0, 0.0, 0.0, []
    with threadpool_limits(1):
        t0 = time.perf_counter()
        slots = oracle.slot_mapping(table, lens - 1, bs)
        if fp8:
            oracle.kv_append_fp8(*pools, snap["kn"], snap["vn"], slots, bs, dt, layout, fmt)
        else:
            oracle.kv_append(pools[0], pools[1], snap["kn"], snap["vn"], slots, bs, layout)
        t_total = time.perf_counter() - t0
        for b in range(B):
            if done >= min(B, min_seqs) and t_total >= budget_s:
                break
            t = time.perf_counter()
            if fp8:
                ref = oracle.decode_attention_fp8(snap["q"], *pools, table, lens, cfg.scale, Hkv, bs, dt, seqs=[b],
                                                  layout=layout, fmt=fmt)[b]
            else:
                ref = oracle.decode_attention(snap["q"], pools[0], pools[1], table, lens, cfg.scale, Hkv, bs, dt,
                                              seqs=[b], layout=layout)[b]
            t_total += time.perf_counter() - t
            done += 1
            kv_bytes += 2 * Hkv * row_bytes * int(lens[b])
            got = oracle.upcast(out0[b], dt)
            err = np.abs(got - ref)
            ratio = float(np.max(err / (atol + rtol * np.abs(ref)))) if err.size else 0.0
            if not np.isfinite(got).all() or not ratio <= 1.0:
                bad.append(b)
            worst, worst_ratio = max(worst, float(np.nanmax(err))), max(worst_ratio, ratio)
    append_exact = all(a.tobytes() == p.tobytes() for a, p in zip(after, pools))
    return dict(done=done, kv_bytes=kv_bytes, t=t_total, max_abs_err=worst, max_err_over_tol=worst_ratio,
                bad_seqs=bad, append_bit_exact=append_exact, tol=f"|gpu - ref| <= {atol:g} + {rtol:g} |ref|")


def time_stream(pkv, torch, wkd, L, fp8, lay, pb, kcache0, stream, args, step_kv):
    """Read ceiling of the decode access pattern: every tile the decode launches
    read, in their order, with nothing computed (same pools, tables and
    partitions); ms per L-layer step and GB/s of K/V."""
    sink = pkv.stream_sink(kcache0, wkd.block_tables, pb, layout=lay)

    def stream_step():
        for l in range(L):
            if fp8:
                pkv.stream_tiles(wkd.k_codes[l], wkd.v_codes[l], wkd.block_tables, wkd.context_lens_dev, pb, sink,
                                 wkd.k_scales[l], wkd.v_scales[l], layout=lay)
            else:
                pkv.stream_tiles(wkd.k_cache[l], wkd.v_cache[l], wkd.block_tables, wkd.context_lens_dev, pb, sink,
                                 layout=lay)

    for _ in range(max(1, args.warmup)):
        stream_step()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(args.steps):
        stream_step()
    s1.record(stream)
    torch.cuda.synchronize()
    stream_ms = s0.elapsed_time(s1) / args.steps
    stream_gbs = step_kv / (stream_ms * 1e-3) / 1e9
    log(f"stream ceiling: {stream_ms:.3f} ms per {L} launches = {stream_gbs:.0f} GB/s of K/V")
    return stream_ms, stream_gbs


def run_copy_blocks(args):
    """--op copy_blocks: copy-on-write block copies at the Llama-3-70B cache
    shape (bf16, 8 KV heads, head_dim 128, 16-token blocks: 32 KiB per block
    per tensor), K and V in one launch, `--copy-pairs` random (src, dst) pairs
    per launch with distinct destinations."""
    import torch
    from paged_kv_cache_156_amd import binding as pkv

    pkv.load()
    dev = torch.device("cuda:0")
    Hkv, D, bs, n = 8, 128, 16, args.copy_pairs
    NB = 2 * n
    g = torch.Generator(device=dev)
    g.manual_seed(156)
    kc = torch.randn((NB, Hkv, bs, D), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((NB, Hkv, bs, D), generator=g, device=dev).to(torch.bfloat16)
    rng = np.random.default_rng(156)
    pairs_h = np.stack([rng.permutation(n), n + rng.permutation(n)], 1).astype(np.int32)  # sources, then fresh blocks
    pairs = torch.from_numpy(pairs_h).to(dev)
    block_bytes = Hkv * bs * D * 2
    bytes_launch = 2 * 2 * block_bytes * n  # K and V, read + write
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pkv.copy_blocks([kc, vc], pairs)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        pkv.copy_blocks([kc, vc], pairs)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    assert torch.equal(kc[pairs[:, 1].long()], kc[pairs[:, 0].long()])
    gbs = bytes_launch / (ms * 1e-3) / 1e9
    # reference: one contiguous device copy of the same bytes (torch's copy
    # kernel), the read + write rate the scattered block copies compare with
    src = torch.empty(bytes_launch // 4, dtype=torch.uint16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(args.steps):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    ref_gbs = bytes_launch / (c0.elapsed_time(c1) / args.steps * 1e-3) / 1e9
    del src, dst
    copy_calibration(args, torch, dev)
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        k_h = kc[: min(n, 4096)].view(torch.int16).cpu().numpy()  # 128 MiB: larger than the host caches
        sample = [(i, i + len(k_h) // 2) for i in range(len(k_h) // 2)]
        done, t_cpu = 0, 0.0
        while t_cpu < min(args.cpu_budget, 5.0):
            t = time.perf_counter()
            oracle.copy_blocks(k_h, sample)
            t_cpu += time.perf_counter() - t
            done += len(sample)
        cpu = {"value": round(2 * block_bytes * done / t_cpu / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} block copies of one 32 KiB tensor block (NumPy, one thread), {t_cpu:.1f}s"}
    result = {
        "metric": "copy-on-write block copy GB/s (bytes read + written)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (bit copy)", "data": "synthetic",
        "config": {"workload": f"copy_blocks: {n} random block pairs, K and V caches of 8 KV heads x 16 tokens x "
                               f"128 dims bf16 (32 KiB per block per tensor), one launch", "pairs": n},
        "roofline": {"bound": "hbm", "kernel": "copy_blocks_kernel", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "alg_bytes_per_launch": bytes_launch, "avg_launch_us": round(ms * 1e3, 2),
                     "kernel_sha": kernel_sha()},
        "contiguous_copy_gbps": round(ref_gbs, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def run_prefill(args):
    """--op prefill: chunked-prefill attention at the Llama-3-70B attention
    shape (64 query / 8 KV heads, head_dim 128, bf16, 16-token blocks):
    `--prefill-seqs` sequences, each with `--prefill-context` cached tokens
    followed by a chunk of `--prefill-chunk` new query tokens (their K/V
    already appended). FLOPs counted: 4 * Hq * D per (query token, visible
    key) pair -- QK^T and PV -- over the causal triangle."""
    import torch
    from paged_kv_cache_156_amd import binding as pkv
    from paged_kv_cache_156_amd import workloads as wl

    pkv.load()
    dev = torch.device("cuda:0")
    B, C, P = args.prefill_seqs, args.prefill_chunk, args.prefill_context
    base = wl.CONFIG_BY_NAME["llama3_70b"]
    cfg = dataclasses.replace(base, name="prefill_70b", num_seqs=B, context_lens=(P + C,) * B,
                              block_size=args.block_size or 16)
    Hq, Hkv, D, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    lens = np.full(B, P + C, np.int32)
    asg, slots, _ = pool_assignment(cfg, lens, pkv, wl)
    q8 = args.kv != "native"
    fmt = "int8" if args.kv == "int8" else "e4m3"
    nhd = (lambda x: x.transpose(1, 2).contiguous()) if args.layout == "NHD" else (lambda x: x)
    slots_d = torch.from_numpy(slots).to(dev)
    if q8:  # 8-bit codes + per-row scales (the values are random codes)
        wkd = wl.make_device_workload_fp8(cfg, dev, layers=1, context_lens=lens, assignment=asg)
        kc, vc = nhd(wkd.k_codes[0]), nhd(wkd.v_codes[0])
        ks, vs = nhd(wkd.k_scales[0]), nhd(wkd.v_scales[0])
        pkv.kv_append_fp8(wkd.k_new[0], wkd.v_new[0], slots_d, kc, vc, ks, vs, layout=args.layout, fmt=fmt)
    else:
        wkd = wl.make_device_workload(cfg, dev, layers=1, context_lens=lens, assignment=asg)
        kc, vc = nhd(wkd.k_cache[0]), nhd(wkd.v_cache[0])
        # the last position too: every chunk token's K/V is in the cache
        pkv.kv_append(wkd.k_new[0], wkd.v_new[0], slots_d, kc, vc, layout=args.layout)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    q = torch.randn((B * C, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    q_start = torch.arange(0, B * C + 1, C, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    pb = args.partition_blocks
    ws = pkv.alloc_prefill_workspace(q_start, Hq, kc, wkd.block_tables, C, pb, layout=args.layout)

    def launch():
        if q8:
            pkv.prefill_attention_fp8(q, kc, vc, ks, vs, wkd.block_tables, q_start, C, wkd.context_lens_dev, cfg.scale,
                                      out, ws, pb, layout=args.layout, fmt=fmt)
        else:
            pkv.prefill_attention(q, kc, vc, wkd.block_tables, q_start, C, wkd.context_lens_dev, cfg.scale, out, ws,
                                  pb, layout=args.layout)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item(), "non-finite prefill output"
    settle_ms = 200.0 if args.settle_ms is None else args.settle_ms
    settled = settle(launch, torch, settle_ms)
    log(f"settle: {settled} untimed launches over {settle_ms:.0f} ms")
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        launch()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    copy_calibration(args, torch, dev)
    pairs = B * sum(P + i + 1 for i in range(C))  # (query token, visible key) pairs
    flops = 4 * Hq * D * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        import time as _t
        # one sequence's chunk, the first rows only, on the host
        blocks = asg.blocks[0]
        idx = torch.from_numpy(blocks.astype(np.int64)).to(dev)
        if q8:
            kh, vh, ksh, vsh = (x.index_select(0, idx).cpu().numpy() for x in (kc, vc, ks, vs))
        else:
            kh = wl.torch_to_raw(kc.index_select(0, idx), "bf16")
            vh = wl.torch_to_raw(vc.index_select(0, idx), "bf16")
        qh = wl.torch_to_raw(q[:C], "bf16")
        table = np.arange(len(blocks), dtype=np.int32)[None, :]
        from threadpoolctl import threadpool_limits
        rows, spent, pairs_cpu = 1, 0.0, 0
        nt = 1  # the reference attends row by row in Python; BLAS is held to one thread
        with threadpool_limits(nt):
            while spent < min(args.cpu_budget, 10.0) and rows <= C:
                t = _t.perf_counter()
                if q8:
                    oracle.prefill_attention_fp8(qh[:rows], kh, vh, ksh, vsh, table, [0, rows], [P + rows], cfg.scale,
                                                 Hkv, bs, "bf16", args.layout, fmt=fmt)
                else:
                    oracle.prefill_attention(qh[:rows], kh, vh, table, [0, rows], [P + rows], cfg.scale, Hkv, bs,
                                             "bf16", args.layout)
                spent = _t.perf_counter() - t
                pairs_cpu = sum(P + i + 1 for i in range(rows))
                rows *= 2
        cpu = {"value": round(4 * Hq * D * pairs_cpu / spent / 1e12, 6), "unit": "TFLOP/s", "cores": nt,
               "kind": "oracle", "sample": f"{rows // 2} query tokens of one sequence's chunk, fp64 NumPy on one "
                                           f"thread, {spent:.1f}s"}
    result = {
        "metric": "chunked-prefill paged attention TFLOP/s (QK^T + PV over the causal triangle)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"ms": settle_ms, "launches": settled}, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"{fmt} K/V + f32 row scales, bf16 q/out" if q8 else "bf16", "data": "synthetic",
        "config": {"workload": f"prefill: {B} sequences x {C}-token chunks after {P} cached tokens, 64 query / 8 KV "
                               f"heads, head_dim 128, {args.layout} blocks of {bs}", "seqs": B, "chunk": C,
                   "context": P, "partition_blocks": pb, "kv": args.kv},
        "roofline": {"bound": "mfma", "kernel": "prefill_lds_kernel",
                     "achieved": round(tflops, 2),
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "alg_flops_per_launch": flops, "avg_launch_us": round(ms * 1e3, 2), "kernel_sha": kernel_sha()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 30 timed steps (about 200 ms on the 70B shape), after the settle phase below: a slow
    # stretch of a few ms then weighs less in the mean than over 10 steps
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=None,
                    help="after the warm-up, repeat the step (or launch) untimed for this long before the timed "
                         "steps (default 200: launches reach their sustained rate after some ms of work)")
    ap.add_argument("--config", default="llama3_70b")
    ap.add_argument("--layers", type=int, default=0, help="layers to loop (0 = the configuration's count)")
    ap.add_argument("--partition-blocks", type=int, default=0, help="blocks per partition (0 = library choice)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of CPU-reference work (0 = skip)")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed timing of the same steps")
    ap.add_argument("--mode", choices=("fused", "split"), default="fused",
                    help="fused: one decode_step launch per layer (append + attention + merge); "
                         "split: kv_append, decode_partitions, decode_merge")
    ap.add_argument("--kv", choices=("native", "fp8", "int8"), default="native",
                    help="native: K/V cached in the configuration's dtype; fp8: E4M3 codes + fp32 per-row scales; "
                         "int8: INT8 codes + fp32 per-row scales")
    ap.add_argument("--layout", choices=("HND", "NHD"), default="HND",
                    help="cache block layout: HND [NB, Hkv, bs, D] (default) or NHD [NB, bs, Hkv, D]")
    ap.add_argument("--block-size", type=int, default=0, help="tokens per cache block (0 = the configuration's, 16)")
    ap.add_argument("--op", choices=("decode", "stream", "copy_blocks", "prefill"), default="decode",
                    help="decode: the decode step (default); stream: the read ceiling of the decode access pattern "
                         "(the same tiles, nothing computed); copy_blocks: copy-on-write block copies; "
                         "prefill: chunked-prefill attention")
    ap.add_argument("--prefill-seqs", type=int, default=4)
    ap.add_argument("--prefill-chunk", type=int, default=512)
    ap.add_argument("--prefill-context", type=int, default=4096)
    ap.add_argument("--copy-pairs", type=int, default=8192, help="block pairs per copy_blocks launch")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the decode path runs on one GPU; --gpus must be 1 (there is no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)

    if args.op == "copy_blocks":
        run_copy_blocks(args)
        return
    if args.op == "prefill":
        run_prefill(args)
        return

    import torch
    from paged_kv_cache_156_amd import binding as pkv
    from paged_kv_cache_156_amd import workloads as wl

    pkv.load()
    dev = torch.device("cuda:0")
    cfg = wl.CONFIG_BY_NAME[args.config]
    if args.block_size:
        cfg = dataclasses.replace(cfg, block_size=args.block_size)
    lay = args.layout
    L = args.layers or cfg.num_layers
    _, _, r_len = wl.streams(cfg.seed)
    lens = wl.draw_context_lens(cfg, r_len)
    B, Hq, Hkv, D, bs = len(lens), cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    esz = wl.DTYPE_BYTES[cfg.dtype]

    log(f"config {cfg.name}: B={B} Hq={Hq} Hkv={Hkv} D={D} {cfg.dtype} layers={L} sum(ctx)={int(lens.sum())}")
    asg, slots, pool_stats = pool_assignment(cfg, lens, pkv, wl)
    log(f"block pool: {pool_stats}")
    t0 = time.time()
    fp8 = args.kv in ("fp8", "int8")  # 8-bit codes with per-row scales
    fmt = "int8" if args.kv == "int8" else "e4m3"
    if fp8:
        wkd = wl.make_device_workload_fp8(cfg, dev, layers=L, context_lens=lens, assignment=asg)
    else:
        wkd = wl.make_device_workload(cfg, dev, layers=L, context_lens=lens, assignment=asg,
                                      progress=lambda l: (l % 20 == 0) and log(f"  drew layer {l}/{L}"))
    if lay == "NHD":  # token-major copies of the same caches, one layer at a time
        for l in range(L):
            if fp8:
                wkd.k_codes[l] = wkd.k_codes[l].transpose(1, 2).contiguous()
                wkd.v_codes[l] = wkd.v_codes[l].transpose(1, 2).contiguous()
                wkd.k_scales[l] = wkd.k_scales[l].transpose(1, 2).contiguous()
                wkd.v_scales[l] = wkd.v_scales[l].transpose(1, 2).contiguous()
            else:
                wkd.k_cache[l] = wkd.k_cache[l].transpose(1, 2).contiguous()
                wkd.v_cache[l] = wkd.v_cache[l].transpose(1, 2).contiguous()
    torch.cuda.synchronize()
    log(f"device workload ready in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated)")

    snap = snapshot_layer0(wkd, fp8, cfg.dtype) if (args.cpu_budget > 0 and args.op == "decode") else None

    max_blocks = wkd.block_tables.shape[1]
    pb = args.partition_blocks or pkv.decode_partition_blocks(B, Hq, Hkv, max_blocks, bs)
    fused = args.mode == "fused"
    kcache0 = wkd.k_codes[0] if fp8 else wkd.k_cache[0]
    if fused:
        ws = pkv.alloc_step_workspace(wkd.q[0], kcache0, wkd.block_tables, pb, layout=lay)
    else:
        ws = pkv.alloc_workspace(wkd.q[0], kcache0, wkd.block_tables, pb, layout=lay)
    slots_d = torch.from_numpy(slots).to(dev)
    outs = [torch.empty_like(wkd.q[l]) for l in range(L)]
    stream = torch.cuda.current_stream()
    # K/V bytes read per layer (8-bit caches: codes + one fp32 scale per row)
    # and the algorithmic bytes of one launch
    kv_layer, part_alg = decode_alg_bytes(lens, Hq, Hkv, D, esz, bs, fp8, fused)
    step_kv = kv_layer * L

    if args.op == "stream":
        stream_ms, stream_gbs = time_stream(pkv, torch, wkd, L, fp8, lay, pb, kcache0, stream, args, step_kv)
        copy_calibration(args, torch, dev)
        geom = "" if (lay == "HND" and bs == 16) else f"_{lay.lower()}_bs{bs}"
        traffic = profile_traffic(f"stream{'_' + args.kv if fp8 else ''}{geom}_{cfg.name}_traffic.json", pb)
        print(json.dumps({
            "metric": "decode access-pattern read ceiling GB/s (K/V tiles through the block tables, nothing computed)",
            "value": round(stream_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(stream_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": f"{fmt} codes + f32 row scales" if fp8 else cfg.dtype, "data": "synthetic",
            "config": {"workload": f"{cfg.name}: the tiles of {L} decode launches ({lay} blocks of {bs}, partitions "
                                   f"of {pb} blocks)", "layers": L, "partition_blocks": pb, "kv": args.kv,
                       "layout": lay, "block_size": bs},
            "frac_of_hbm_peak": round(stream_gbs / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": "stream_tiles_kernel", "achieved": round(stream_gbs, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(stream_gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic, "alg_bytes_per_launch": kv_layer,
                         "avg_launch_us": round(stream_ms / L * 1e3, 2), "kernel_sha": kernel_sha()},
            "cpu_baseline": None}), flush=True)
        return

    def step(events=None):
        for l in range(L):
            if fp8:
                if events is not None:
                    events[l][0].record(stream)
                if fused:
                    pkv.decode_step_fp8(wkd.q[l], wkd.k_new[l], wkd.v_new[l], wkd.k_codes[l], wkd.v_codes[l],
                                        wkd.k_scales[l], wkd.v_scales[l], wkd.block_tables, wkd.context_lens_dev,
                                        cfg.scale, outs[l], ws, pb, layout=lay, fmt=fmt)
                else:
                    pkv.kv_append_fp8(wkd.k_new[l], wkd.v_new[l], slots_d, wkd.k_codes[l], wkd.v_codes[l],
                                      wkd.k_scales[l], wkd.v_scales[l], layout=lay, fmt=fmt)
                    pkv.paged_decode_attention_fp8(wkd.q[l], wkd.k_codes[l], wkd.v_codes[l], wkd.k_scales[l],
                                                   wkd.v_scales[l], wkd.block_tables, wkd.context_lens_dev,
                                                   cfg.scale, outs[l], ws, pb, layout=lay, fmt=fmt)
                if events is not None:
                    events[l][1].record(stream)
                continue
            if fused:
                if events is not None:
                    events[l][0].record(stream)
                pkv.decode_step(wkd.q[l], wkd.k_new[l], wkd.v_new[l], wkd.k_cache[l], wkd.v_cache[l],
                                wkd.block_tables, wkd.context_lens_dev, cfg.scale, outs[l], ws, pb, layout=lay)
                if events is not None:
                    events[l][1].record(stream)
                continue
            pkv.kv_append(wkd.k_new[l], wkd.v_new[l], slots_d, wkd.k_cache[l], wkd.v_cache[l], layout=lay)
            if events is not None:
                events[l][0].record(stream)
            pkv.decode_partitions(wkd.q[l], wkd.k_cache[l], wkd.v_cache[l], wkd.block_tables, wkd.context_lens_dev,
                                  cfg.scale, outs[l], ws, pb, layout=lay)
            if events is not None:
                events[l][1].record(stream)
            pkv.decode_merge(wkd.q[l], wkd.k_cache[l], wkd.v_cache[l], wkd.block_tables, wkd.context_lens_dev,
                             outs[l], ws, pb, layout=lay)

    log(f"warmup {args.warmup} steps (partition_blocks={pb}, workspace {0 if ws is None else ws.numel()} B)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert all(torch.isfinite(o).all().item() for o in outs[:2]), "non-finite attention output"
    settle_ms = 200.0 if args.settle_ms is None else args.settle_ms
    settled = settle(step, torch, settle_ms)
    log(f"settle: {settled} untimed steps over {settle_ms:.0f} ms")

    # timed region: K steps back to back, bracketed by events on the launch stream
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # the same K steps again with an event pair around every launch of the
    # dominant kernel, for its average launch duration
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
              for _ in range(args.steps)]
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    part_ms = [ev[l][0].elapsed_time(ev[l][1]) for ev in events for l in range(L)]
    event_avg_ms = float(np.mean(part_ms))
    # and once more with an event pair around every step: median and minimum
    step_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        step_ev[k][0].record(stream)
        step()
        step_ev[k][1].record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    # The same step captured once into a HIP graph and replayed K times: the
    # kernels are the same; the graph removes the host launch path between
    # them. Reported beside the eager figures, which stay the headline.
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        assert all(torch.isfinite(o).all().item() for o in outs[:2]), "non-finite attention output after replay"
        del g
        log(f"graph replay: {graph_ms:.3f} ms/step")
    # In fused mode the step is exactly one launch of the kernel per layer, so
    # the timed region's events give its average launch duration directly (an
    # event pair around each launch adds several microseconds of its own).
    part_avg_ms = total_ms / (args.steps * L) if fused else event_avg_ms
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; partition kernel avg {part_avg_ms * 1e3:.1f} us")

    gbs = step_kv / (ms_per_step * 1e-3) / 1e9
    achieved = part_alg / (part_avg_ms * 1e-3) / 1e9

    geom = "" if (lay == "HND" and bs == 16) else f"_{lay.lower()}_bs{bs}"
    traffic = profile_traffic(f"decode_{args.mode}{'_' + args.kv if fp8 else ''}{geom}_{cfg.name}_traffic.json", pb)

    stream_ms, stream_gbs = time_stream(pkv, torch, wkd, L, fp8, lay, pb, kcache0, stream, args, step_kv)

    cpu, parity = None, None
    if snap is not None:
        log("CPU reference on layer 0 (append, then attention sequence by sequence) and comparison ...")
        chk = oracle_check(snap, wl.torch_to_raw(outs[0], cfg.dtype), pools_after(wkd, fp8, cfg.dtype), cfg, lay,
                           fp8, fmt, args.cpu_budget)
        cpu = {"value": round(chk["kv_bytes"] / chk["t"] / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "seqs_per_s": round(chk["done"] / (chk["t"] * L), 4),
               "sample": f"layer 0 of {cfg.name}: the new token of all {B} sequences appended into the whole pool, "
                         f"then attention for the first {chk['done']} sequences through the same block tables, "
                         f"fp64 NumPy on one thread (a per-token Python gather), {chk['t']:.1f}s; seqs/s "
                         f"extrapolated to {L} layers"}
        parity = {"checked_seqs": chk["done"], "of_seqs": B, "max_abs_err": chk["max_abs_err"],
                  "max_err_over_tol": round(chk["max_err_over_tol"], 4), "tol": chk["tol"],
                  "append_bit_exact": chk["append_bit_exact"], "bad_seqs": chk["bad_seqs"][:16],
                  "ok": chk["append_bit_exact"] and not chk["bad_seqs"]}
        log(f"cpu baseline: {cpu}")
        log(f"parity against the CPU reference: {parity}")

    # bytes of distinct cache rows read (shared prefix blocks counted once)
    rows_seen = {}
    for b, n in enumerate(lens):
        for lb, pbk in enumerate(asg.blocks[b][: -(-int(n) // bs)]):
            rows_seen[int(pbk)] = max(rows_seen.get(int(pbk), 0), min(bs, int(n) - lb * bs))
    unique_tokens = sum(rows_seen.values())
    unique_layer = 2 * Hkv * ((D + 4) if fp8 else D * esz) * unique_tokens

    copy_calibration(args, torch, dev)

    result = {
        "metric": "paged decode attention K/V-read GB/s (% of HBM peak) and seqs/s at 1 GPU",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": settle_ms, "steps": settled},
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(np.min(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"{fmt} K/V + f32 row scales, {cfg.dtype} q/out" if fp8 else cfg.dtype),
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: batch {B}, context {'ragged' if cfg.context_len_range else int(lens[0])}, "
                               f"{Hq} query / {Hkv} KV heads, head_dim {D}, {lay} blocks of {bs}, {L} layers, one decode step "
                               f"(append + attention) per layer",
                   "global_batch": B, "seq_len": int(lens.max()), "layers": L, "partition_blocks": pb,
                   "mode": args.mode, "kv": args.kv, "layout": lay, "block_size": bs},
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "stream_ceiling_gbps": round(stream_gbs, 2),
        "frac_of_stream_ceiling": round(gbs / stream_gbs, 4),
        "seqs_per_s": round(B / (ms_per_step * 1e-3), 2),
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 4), "value": round(step_kv / (graph_ms * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(step_kv / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(graph_ms / L * 1e3, 2),
            "note": "the same steps captured into one HIP graph and replayed; value above is the eager stream"},
        "kv_bytes_per_step": step_kv,
        "unique_kv_bytes_per_step": unique_layer * L,
        "unique_kv_gbps": round(unique_layer * L / (ms_per_step * 1e-3) / 1e9, 2),
        "parity_checked_seqs": parity["checked_seqs"] if parity else 0,
        "parity": parity,
        "roofline": {"bound": "hbm", "kernel": "decode_partition_kernel<" + ("step" if fused else "split") + ">",
                     "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": part_alg,
                     "avg_launch_us": round(part_avg_ms * 1e3, 2),
                     "avg_launch_us_per_launch_events": round(event_avg_ms * 1e3, 2),
                     "kernel_sha": kernel_sha()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    if parity is not None and not parity["ok"]:
        log(f"PARITY FAILURE: {parity}")
        sys.exit(1)


if __name__ == "__main__":
    main()
