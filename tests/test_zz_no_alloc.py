"""GPU test of pkv_decode_step_noalloc (the fused step with the library's own
static scratch instead of a caller workspace), through the C ABI: two calls in
a row, the second with a smaller input, each checked against pkv_decode_step
with a workspace (bit for bit: same kernels, same partitions) and against the
CPU reference at the attention tolerance; the appended caches byte for byte."""
import sys

import numpy as np
import pytest

import oracle
from paged_kv_cache_156_amd import binding as pkv
from paged_kv_cache_156_amd import workloads as wl

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(torch, dev, wk, pb):
    """The workspace entry point and the no-allocation one on fresh copies of
    the same inputs; returns both outputs and caches (raw host arrays)."""
    cfg = wk.cfg
    dt = cfg.dtype
    t = torch.from_numpy(np.ascontiguousarray(wk.block_tables, np.int32)).to(dev)
    lens = torch.from_numpy(wk.context_lens.astype(np.int32)).to(dev)
    q = wl.raw_to_torch(wk.q, dt, dev)
    kn, vn = wl.raw_to_torch(wk.k_new, dt, dev), wl.raw_to_torch(wk.v_new, dt, dev)
    res = []
    for noalloc in (False, True):
        kc, vc = wl.raw_to_torch(wk.k_cache, dt, dev), wl.raw_to_torch(wk.v_cache, dt, dev)
        out = torch.full_like(q, float("nan"))
        if noalloc:
            pkv.decode_step_noalloc(q, kn, vn, kc, vc, t, lens, cfg.scale, out, pb)
        else:
            ws = pkv.alloc_step_workspace(q, kc, t, pb)
            pkv.decode_step(q, kn, vn, kc, vc, t, lens, cfg.scale, out, ws, pb)
        torch.cuda.synchronize()
        res.append((wl.torch_to_raw(out, dt), wl.torch_to_raw(kc, dt), wl.torch_to_raw(vc, dt)))
    return res


def check_against_reference(wk, out):
    cfg = wk.cfg
    kc, vc = wk.k_cache.copy(), wk.v_cache.copy()
    oracle.kv_append(kc, vc, wk.k_new, wk.v_new, oracle.slot_mapping(wk.block_tables, wk.context_lens - 1, 16), 16)
    ref = oracle.decode_attention(wk.q, kc, vc, wk.block_tables, wk.context_lens, cfg.scale, cfg.num_kv_heads, 16,
                                  cfg.dtype)
    atol, rtol = (1e-5, 1e-5) if cfg.dtype == "f32" else (2e-3, 1e-2)
    got = oracle.upcast(out, cfg.dtype)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= atol + rtol * np.abs(ref)).all()
    return kc, vc


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load()
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_step_matches_workspace_step_twice(torch_dev, dtype):
    torch, dev = torch_dev
    big = wl.DecodeConfig("noalloc_big", 0, 1, 12, 32, 8, 128, 16, dtype,
                          context_lens=(1, 17, 300, 1000, 2049, 4096, 64, 513, 3000, 16, 777, 1500))
    small = wl.DecodeConfig("noalloc_small", 0, 1, 3, 8, 2, 64, 16, dtype, context_lens=(40, 5, 300))
    for cfg, pb, seed in ((big, 8, 11), (small, 1, 12)):  # second call: smaller input, other partitions
        note(f"no-alloc step {dtype}: {cfg.name} (B={cfg.num_seqs}, pb={pb})")
        wk = wl.make_host_workload(cfg, seed=seed)
        (o_ws, k_ws, v_ws), (o_na, k_na, v_na) = run_both(torch, dev, wk, pb)
        assert o_na.tobytes() == o_ws.tobytes(), f"{cfg.name}: outputs differ from the workspace entry point"
        kc_o, vc_o = check_against_reference(wk, o_na)
        assert k_na.tobytes() == kc_o.tobytes() and v_na.tobytes() == vc_o.tobytes()
        assert k_ws.tobytes() == kc_o.tobytes() and v_ws.tobytes() == vc_o.tobytes()


def test_noalloc_step_rejects_shapes_beyond_its_array(torch_dev):
    torch, dev = torch_dev
    # 32768-token contexts in partitions of one block: 2048 partitions x 64 units of partials, > 64 MiB
    B, Hq, Hkv, D, mb = 8, 64, 8, 128, 2048
    assert pkv.decode_step_workspace_bytes(B, Hq, Hkv, D, mb, 1) > (64 << 20)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((16, Hkv, 16, D), dtype=torch.bfloat16, device=dev)
    t = torch.zeros((B, mb), dtype=torch.int32, device=dev)
    lens = torch.ones((B,), dtype=torch.int32, device=dev)
    kn = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device=dev)
    with pytest.raises(pkv.PkvError) as e:
        pkv.decode_step_noalloc(q, kn, kn, kc, kc, t, lens, 0.1, torch.empty_like(q), 1)
    assert e.value.status == pkv.PKV_ESMALL
