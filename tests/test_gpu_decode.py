"""GPU: pa_decode against the float64 CPU oracle, element by element.

Tolerances are max-abs 1e-5 (fp32), 2e-3 (fp16), 1e-2 (bf16) on every output element.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_indexed_amd import ops
from paged_kv_cache_indexed_amd._lib import (PA_FLAG_BAD_BLOCK_ID, PA_FLAG_BAD_LENGTH,
                                             PA_FLAG_EMPTY_CONTEXT, CacheDesc,
                                             pa_decode_partition_size)
from tests.gpu_util import TOL, assert_close, gpu_decode, note, oracle_decode, require_gpu
from workloads import build_paged, config_workload

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ shapes, dtypes, groups

_SWEEP = [(dt, d, g) for dt in ("f32", "f16", "bf16") for d in (64, 128, 256)
          for g in (1, 2, 4, 8, 16) if not (g == 16 and d == 256)]


@pytest.mark.parametrize("dtype,head_dim,group", _SWEEP, ids=lambda x: str(x))
def test_dtype_headdim_group(dtype, head_dim, group):
    dev = require_gpu()
    lens = np.array([1, 7, 16, 17, 100, 250], np.int32)
    w = build_paged(f"sweep-{dtype}-{head_dim}-{group}", 100 + group, head_dim, lens, 16, 2,
                    2 * group, head_dim, dtype)
    ref = oracle_decode(w)
    t = w.to_device(dev)
    for P in (0, 32, 128):
        note(f"sweep dtype={dtype} d={head_dim} G={group} P={P}")
        got, _ = gpu_decode(w, dev, partition_size=P, tensors=t)
        assert_close(got, ref, dtype, f"sweep {dtype} d={head_dim} G={group} P={P}")


@pytest.mark.parametrize("bs", [8, 16, 32, 64, 128, 256, 512])
def test_block_sizes(bs):
    dev = require_gpu()
    lens = np.array([1, bs - 1, bs, bs + 1, 3 * bs + 5, 600], np.int32)
    w = build_paged(f"bs{bs}", 200, bs, lens, bs, 4, 4, 128, "f16")
    ref = oracle_decode(w)
    t = w.to_device(dev)
    for P in (0, bs * max(1, 64 // bs), bs * 4):
        note(f"block size {bs} P={P}")
        got, _ = gpu_decode(w, dev, partition_size=P, tensors=t)
        assert_close(got, ref, "f16", f"bs={bs} P={P}")


_GQA8 = [(dt, d, g) for dt in ("f16", "bf16") for d in (64, 128) for g in (4, 8, 16)]


@pytest.mark.parametrize("dtype,head_dim,group", _GQA8, ids=lambda x: str(x))
def test_grouped_heads_8_token_blocks(dtype, head_dim, group):
    """Grouped heads over 8-token blocks run on the matrix cores, a 16-row tile spanning two
    blocks (16-bit rows of 128 dims: one buffer over both blocks; otherwise per-lane row
    addresses). Unused slots hold NaN; partitions of 8 and 24 tokens start in the middle of
    a tile."""
    dev = require_gpu()
    lens = np.array([1, 7, 8, 9, 15, 16, 17, 100, 250, 600], np.int32)
    w = build_paged(f"gqa-bs8-{dtype}-{head_dim}-{group}", 300 + group, head_dim, lens, 8, 2, 2 * group,
                    head_dim, dtype)
    ref = oracle_decode(w)
    t = w.to_device(dev)
    for P in (0, 8, 24, 64, 512, 2048):
        note(f"grouped heads bs=8 dtype={dtype} d={head_dim} G={group} P={P}")
        got, _ = gpu_decode(w, dev, partition_size=P, tensors=t)
        assert_close(got, ref, dtype, f"bs=8 {dtype} d={head_dim} G={group} P={P}")


@pytest.mark.parametrize("group", [8, 16])
def test_grouped_heads_8_token_blocks_far_apart(group):
    """A tile's two 8-token blocks more than 2 GiB apart in the pool (every other block of a
    sequence moved up by 600000 ids, 2.3 GiB per pool). With 8 heads per kv head the LDS path
    gives each 4-row load its own block's buffer; with 16 the direct-load kernel loads the two
    8-row halves from their own blocks through per-lane addresses."""
    dev = require_gpu()
    lens = np.array([1, 9, 100, 250], np.int32)
    w = build_paged("gqa-bs8-far", 320, 0, lens, 8, 2, 2 * group, 128, "bf16")
    ref = oracle_decode(w)
    far = 600_000
    tab = w.block_table.copy()
    odd = np.zeros_like(tab, dtype=bool)
    odd[:, 1::2] = True
    tab = np.where((tab >= 0) & odd, tab + far, tab).astype(np.int32)
    used = np.unique(w.block_table[w.block_table >= 0])
    t = w.to_device(dev)
    shape = (far + w.num_blocks, 2, 8, 128)
    kp = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    vp = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    ids = torch.from_numpy(np.where(np.isin(used, w.block_table[:, 1::2]), used + far, used)).long().to(dev)
    src = torch.from_numpy(used).long().to(dev)
    kp[ids] = t["k_pool"][src]
    vp[ids] = t["v_pool"][src]
    tt = torch.from_numpy(tab).to(dev)
    for P in (0, 16, 2048):
        note(f"grouped heads bs=8 G={group}, blocks 2.3 GiB apart, P={P}")
        out = ops.decode(t["q"], kp, vp, tt, t["context_lens"], int(lens.max()), w.scale, partition_size=P)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy().astype(np.float64), ref, "bf16", f"far blocks P={P}")
    del kp, vp


# ------------------------------------------------------------------ the five workloads

def test_config1_decode_append_decode():
    dev = require_gpu()
    w = config_workload(1, seed=0)
    t = w.to_device(dev)
    note("config 1 decode at L")
    got, _ = gpu_decode(w, dev, tensors=t)
    assert_close(got, oracle_decode(w), "f32", "config 1 before append")
    note("config 1 append")
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], t["slot_mapping"])
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    assert np.array_equal(t["k_pool"].cpu().numpy(), ek, equal_nan=True)
    assert np.array_equal(t["v_pool"].cpu().numpy(), ev, equal_nan=True)
    note("config 1 decode at L+1")
    got, _ = gpu_decode(w, dev, lens=w.lens_after_append, tensors=t)
    ref = oracle.paged_decode(w.q, ek, ev, w.block_table, w.lens_after_append, w.scale)
    assert_close(got, ref, "f32", "config 1 after append")


def test_config2_full():
    dev = require_gpu()
    w = config_workload(2, seed=0)
    t = w.to_device(dev)
    ek, ev = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    note("config 2 append")
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], t["slot_mapping"])
    ref = oracle.paged_decode(w.q, ek, ev, w.block_table, w.lens_after_append, w.scale)
    for P in (0, 64, 256, 512):
        note(f"config 2 decode P={P}")
        got, _ = gpu_decode(w, dev, lens=w.lens_after_append, partition_size=P, tensors=t)
        assert_close(got, ref, "f16", f"config 2 P={P}")


@pytest.mark.parametrize("median", [87, 23])
def test_config3_block_size_sweep(median):
    dev = require_gpu()
    outs = {}
    for bs in (8, 16, 32, 64):
        w = config_workload(3, seed=0, block_size=bs, median=median)
        note(f"config 3 median={median} bs={bs} B={w.batch} sumL={int(w.context_lens.sum())}")
        ref = oracle_decode(w)
        got, _ = gpu_decode(w, dev)
        assert_close(got, ref, "f16", f"config 3 med={median} bs={bs}")
        outs[bs] = got
        nb = int(sum(-(-int(L) // bs) for L in w.context_lens))
        waste = 1.0 - float(w.context_lens.sum()) / (nb * bs)
        print(f"[gpu-result] config 3 med={median} bs={bs} padding waste {100 * waste:.1f}%")
        del w
    for bs in (16, 32, 64):
        assert np.max(np.abs(outs[bs] - outs[8])) <= TOL["f16"], "block sizes disagree"


@pytest.mark.parametrize("bs", [8, 16, 256])
def test_config4_gqa(bs):
    dev = require_gpu()
    w = config_workload(4, seed=0, block_size=bs)
    t = w.to_device(dev)
    ek, ev = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], t["slot_mapping"])
    ref = oracle.paged_decode(w.q, ek, ev, w.block_table, w.lens_after_append, w.scale)
    for P in (0, 512):
        note(f"config 4 bs={bs} P={P}")
        got, _ = gpu_decode(w, dev, lens=w.lens_after_append, partition_size=P, tensors=t)
        assert_close(got, ref, "bf16", f"config 4 bs={bs} P={P}")


# ------------------------------------------------------------------ paging invariants

def test_physical_relabel_is_bitwise_invariant():
    dev = require_gpu()
    w = config_workload(2, seed=1, batch=16, heads=4)
    rng = np.random.default_rng(5)
    pi = rng.permutation(w.num_blocks)
    kp2 = np.empty_like(w.k_pool)
    vp2 = np.empty_like(w.v_pool)
    kp2[pi] = w.k_pool
    vp2[pi] = w.v_pool
    t2 = np.where(w.block_table >= 0, pi[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    for P in (0, 64):
        note(f"relabel P={P}")
        a, _ = gpu_decode(w, dev, partition_size=P)
        w2 = dataclasses.replace(w, k_pool=kp2, v_pool=vp2, block_table=t2)
        b, _ = gpu_decode(w2, dev, partition_size=P)
        assert np.array_equal(a, b), "output depends on physical placement"


def test_nan_padding_and_garbage_ids_never_read():
    dev = require_gpu()
    w = config_workload(3, seed=2, batch=24, heads=2, block_size=16)
    clean, _ = gpu_decode(w, dev)
    t = w.to_device(dev)
    tab = w.block_table.copy()
    for b, L in enumerate(w.context_lens):
        n = -(-int(L) // 16)
        tab[b, n:] = np.where(np.arange(tab.shape[1] - n) % 2 == 0, 10 ** 9, -7)
    t["block_table"] = torch.from_numpy(tab).to(dev)
    note("garbage ids past the valid blocks")
    got, _ = gpu_decode(w, dev, tensors=t)
    assert np.all(np.isfinite(got)) and np.array_equal(got, clean)


def test_isolation_between_sequences():
    dev = require_gpu()
    w = config_workload(2, seed=3, batch=8, heads=2)
    base, _ = gpu_decode(w, dev)
    vp = w.v_pool.copy()
    for j in range(-(-int(w.context_lens[0]) // 16)):
        vp[w.block_table[0, j]] *= np.float32(-1.0)
    w.v_pool = vp
    note("isolation")
    got, _ = gpu_decode(w, dev)
    assert np.array_equal(got[1:], base[1:]), "another sequence's output changed"
    assert not np.array_equal(got[0], base[0])
    assert_close(got, oracle_decode(w), "f16", "isolation")


def test_partition_sizes_agree():
    dev = require_gpu()
    w = config_workload(3, seed=4, batch=32, heads=2, block_size=16)
    ref = oracle_decode(w)
    t = w.to_device(dev)
    outs = []
    for P in (16, 64, 512, 4096, 0):
        note(f"partition size {P}")
        got, _ = gpu_decode(w, dev, partition_size=P, tensors=t)
        assert_close(got, ref, "f16", f"P={P}")
        outs.append(got)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= TOL["f16"]


# ------------------------------------------------------------------ errors and edges

@pytest.mark.parametrize("P", [0, 16])
def test_bad_inputs_set_flags_and_nan_only_that_sequence(P):
    dev = require_gpu()
    w = config_workload(2, seed=5, batch=6, heads=2)
    ref = oracle_decode(w)
    t = w.to_device(dev)
    tab = w.block_table.copy()
    tab[1, 3] = w.num_blocks + 11        # bad id inside sequence 1's valid range
    lens = w.context_lens.copy()
    lens[3] = 0                           # empty context
    max_len = int(w.context_lens.max())
    lens[4] = max_len + 1                 # longer than max_context_len
    t["block_table"] = torch.from_numpy(tab).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    # canaries around the output
    buf = torch.full((w.batch * w.num_q_heads * 128 + 2 * 64,), 7.0, dtype=torch.float16, device=dev)
    out = buf[64:64 + w.batch * w.num_q_heads * 128].view(w.batch, w.num_q_heads, 128)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    note(f"bad inputs P={P}")
    ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], lens_t, max_len, w.scale,
               partition_size=P, out=out, err_flag=err)
    torch.cuda.synchronize()
    flags = int(err.item())
    assert flags == PA_FLAG_BAD_BLOCK_ID | PA_FLAG_EMPTY_CONTEXT | PA_FLAG_BAD_LENGTH, flags
    o = out.float().cpu().numpy()
    for b in (1, 3, 4):
        assert np.all(np.isnan(o[b])), f"sequence {b} must be NaN"
    good = [0, 2, 5]
    assert_close(o[good].astype(np.float64), ref[good], "f16", "good sequences beside bad ones")
    assert torch.all(buf[:64] == 7.0) and torch.all(buf[-64:] == 7.0), "canary overwritten"


@pytest.mark.parametrize("dtype,group,P", [("f16", 1, 64), ("f16", 1, 256), ("bf16", 8, 64), ("f32", 2, 32)])
def test_loose_max_context_len(dtype, group, P):
    """max_context_len far above every length: most partitions are past the end of their
    sequence and retire early; the outputs (and a fused append) are unchanged. f16 G=1 P=64
    runs the head-mode kernel, P=256 the split kernel, bf16 G=8 the matrix cores."""
    dev = require_gpu()
    lens = np.array([1, 17, 64, 65, 300, 5, 129, 40], np.int32)
    w = build_paged(f"loose-{dtype}", 310 + group, 0, lens, 16, 2, 2 * group, 128, dtype, max_blocks_per_seq=256)
    ref = oracle_decode(w)
    t = w.to_device(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for max_len in (300, 4096):
        note(f"loose max_context_len={max_len} {dtype} G={group} P={P}")
        out = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"], max_len, w.scale,
                         partition_size=P, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert_close(out.float().cpu().numpy(), ref, dtype, f"max_context_len={max_len} P={P}")
    if dtype == "f32":
        return
    note(f"loose max_context_len fused append {dtype} G={group} P={P}")
    out = ops.decode_append(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"], 4096, w.scale,
                            t["new_key"], t["new_value"], t["slot_mapping"], partition_size=P, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ka, va = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    assert_close(out.float().cpu().numpy(), oracle.paged_decode(w.q, ka, va, w.block_table, w.lens_after_append,
                                                                w.scale), dtype, f"fused, loose bound, P={P}")
    for got, want in zip((t["k_pool"], t["v_pool"]), (ka, va)):
        g = got.float().cpu().numpy()
        assert np.array_equal(np.isnan(g), np.isnan(want)) and np.array_equal(np.nan_to_num(g), np.nan_to_num(want))


def test_max_sizes_and_single_long_partition():
    dev = require_gpu()
    bs = 8
    lens = np.array([8000, 8192, 1, 4097], np.int32)
    w = build_paged("max", 300, 0, lens, bs, 2, 16, 256, "f32", max_blocks_per_seq=1025, append=False)
    ref = oracle_decode(w)
    t = w.to_device(dev)
    for P in (8192, 0, 512):
        note(f"max sizes fp32 d=256 G=8 P={P}")
        got, _ = gpu_decode(w, dev, partition_size=P, tensors=t)
        assert_close(got, ref, "f32", f"max sizes P={P}")


def test_host_argument_checks():
    dev = require_gpu()
    w = config_workload(1, seed=0)
    t = w.to_device(dev)
    c = CacheDesc.of(t["k_pool"])
    assert pa_decode_partition_size(c, 4, 8, 128, 24) == -1  # not a multiple of the block size
    from paged_kv_cache_indexed_amd._lib import PagedKVError
    with pytest.raises(PagedKVError):
        # max_context_len beyond the table's capacity is rejected before any launch
        ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"],
                   w.max_blocks_per_seq * 16 + 1, w.scale)
    with pytest.raises(PagedKVError):
        ops.decode(t["q"][:, :6].contiguous(), t["k_pool"], t["v_pool"], t["block_table"],
                   t["context_lens"], 128, w.scale)  # 6 query heads over 8 kv heads
