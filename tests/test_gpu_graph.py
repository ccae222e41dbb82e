"""GPU: the benchmark step captured in a HIP graph and replayed, against eager launches.

Every replay is checked, with eager work and synchronisation between replays: the pools
and the output of each replay must equal those of the eager step bit for bit (the step is
idempotent: it appends the same token to the same slot)."""

import numpy as np
import pytest
import torch

import oracle.fp8_cache as o8
from paged_kv_cache_indexed_amd import ops
from tests.gpu_util import note, require_gpu
from workloads import config_workload

pytestmark = pytest.mark.gpu

_INT = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16, torch.uint8: torch.uint8}


def _bits(x):
    return x.view(_INT[x.dtype])


@pytest.mark.parametrize("cfg,kw,P", [(2, dict(batch=16, heads=8), 0), (3, dict(batch=64, heads=4), 64),
                                      (4, dict(batch=8), 0)])
def test_fused_step_graph_replays(cfg, kw, P):
    dev = require_gpu()
    w = config_workload(cfg, seed=21, **kw)
    t = w.to_device(dev)
    L = int(w.lens_after_append.max())
    out = torch.empty_like(t["q"])
    ws = ops.workspace_for(t["k_pool"], w.batch, w.num_q_heads, L, P)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()

    def step():
        ops.decode_append(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"], L, w.scale,
                          t["new_key"], t["new_value"], t["slot_mapping"], partition_size=P, out=out, workspace=ws)

    note(f"graph replay cfg={cfg} {kw} P={P}")
    step()
    torch.cuda.synchronize()
    want = [out.clone(), t["k_pool"].clone(), t["v_pool"].clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for k in range(3):
        # eager work between replays: clobber the output, restore the pools to before the append
        out.fill_(float("nan"))
        t["k_pool"].copy_(k0)
        t["v_pool"].copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out, t["k_pool"], t["v_pool"]), want):
            assert torch.equal(_bits(got), _bits(ref)), f"replay {k} differs from the eager step"


def test_fp8_step_graph_replays():
    dev = require_gpu()
    w = config_workload(2, seed=22, batch=16, heads=8)
    t = w.to_device(dev)
    L = int(w.lens_after_append.max())
    # the context rows quantised by the oracle's encoder (unwritten rows: zero codes, zero scales)
    kc, ksc = o8.quantize_rows(np.nan_to_num(w.k_pool))
    vc, vsc = o8.quantize_rows(np.nan_to_num(w.v_pool))
    k8, v8, ks, vs = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (kc, vc, ksc, vsc))
    out = torch.empty_like(t["q"])
    ws = ops.workspace_for(k8, w.batch, w.num_q_heads, L, 64)

    def step():
        ops.reshape_and_cache_fp8(t["new_key"], t["new_value"], k8, v8, ks, vs, t["slot_mapping"])
        ops.decode_fp8(t["q"], k8, v8, ks, vs, t["block_table"], t["lens_after"], L, w.scale, partition_size=64,
                       out=out, workspace=ws)

    note("graph replay fp8 step")
    step()
    torch.cuda.synchronize()
    want = [out.clone(), k8.clone(), ks.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for k in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out, k8, ks), want):
            assert torch.equal(_bits(got), _bits(ref)), f"fp8 replay {k} differs from the eager step"


def test_beam_step_graph_replays():
    """Copy-on-write, append and the beam-group decode of a small beam workload (2 groups of 4
    beams sharing a 2048-token prefix) captured and replayed."""
    from workloads.longctx import beam_workload

    dev = require_gpu()
    w = beam_workload(dev, seed=3, groups=2, beams=4, heads=4, prefix=2048, context=2304)
    t = w.tensors
    L = w.context + 1
    out = torch.empty_like(t["q"])
    n = ops.pa_decode_beams_workspace_bytes(ops.CacheDesc.of(t["k_pool"]), w.batch, w.beams, w.num_q_heads, L, 512)
    ws = torch.empty((n + 3) // 4, dtype=torch.float32, device=dev) if n else None
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()

    def step():
        ops.copy_blocks(t["k_pool"], t["v_pool"], t["copy_pairs"])
        ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], t["slot_mapping"])
        ops.decode_beams(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"], L, w.scale, w.beams,
                         partition_size=512, out=out, workspace=ws)

    note("graph replay beam step")
    step()
    torch.cuda.synchronize()
    want = [out.clone(), t["k_pool"].clone(), t["v_pool"].clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for k in range(3):
        out.fill_(float("nan"))
        t["k_pool"].copy_(k0)
        t["v_pool"].copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out, t["k_pool"], t["v_pool"]), want):
            assert torch.equal(_bits(got), _bits(ref)), f"beam replay {k} differs from the eager step"
