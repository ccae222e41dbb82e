"""GPU: sliding-window decode (pa_decode_sliding_window) against the float64 oracle.

Blocks wholly before each sequence's window are released: their table entries are -1 and
their pool blocks NaN, so any read of them would show.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_indexed_amd import ops
from tests.gpu_util import assert_close, note, require_gpu
from workloads import build_paged, config_workload

pytestmark = pytest.mark.gpu


def _release_before_window(w, window):
    """Table entries and pool blocks wholly before each window: -1 and NaN."""
    tab = w.block_table.copy()
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    for b, L in enumerate(w.context_lens):
        n = max(0, int(L) - window) // w.block_size
        ids = tab[b, :n]
        kp[ids] = np.nan
        vp[ids] = np.nan
        tab[b, :n] = -1
    return dataclasses.replace(w, block_table=tab, k_pool=kp, v_pool=vp)


def _run(w, dev, window, P=0, lens=None):
    t = w.to_device(dev)
    lens_t = t["context_lens"] if lens is None else torch.as_tensor(lens, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], lens_t, int(lens_t.max().item()),
                     w.scale, partition_size=P, err_flag=err, window=window)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f"error flag {int(err.item())}"
    return out.float().cpu().numpy().astype(np.float64), out


@pytest.mark.parametrize("dtype,group,bs", [("f16", 1, 16), ("bf16", 1, 8), ("f32", 2, 16),
                                            ("bf16", 8, 16), ("f16", 4, 32), ("bf16", 8, 8), ("f16", 16, 8)])
def test_window_matches_oracle(dtype, group, bs):
    dev = require_gpu()
    lens = np.array([1, 9, 33, 64, 150, 400], np.int32)
    base = build_paged(f"win-{dtype}", 400 + group, bs, lens, bs, 2, 2 * group, 128, dtype)
    for W in (1, 7, 16, 50, 129, 1000):
        w = _release_before_window(base, W)
        ref = oracle.paged_decode_window(w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.scale, W)
        for P in (0, 2 * bs, 128):
            note(f"window dtype={dtype} G={group} bs={bs} W={W} P={P}")
            got, _ = _run(w, dev, W, P)
            assert_close(got, ref, dtype, f"window {dtype} G={group} W={W} P={P}")


def test_window_at_least_length_equals_full_decode_bitwise():
    dev = require_gpu()
    w = config_workload(3, seed=7, batch=32, heads=4, block_size=16)
    L = int(w.context_lens.max())
    for P in (0, 64):
        note(f"window >= L, P={P}")
        t = w.to_device(dev)
        full = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"], L, w.scale,
                          partition_size=P)
        win = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"], L, w.scale,
                         partition_size=P, window=L)
        torch.cuda.synchronize()
        assert torch.equal(full.view(torch.int16), win.view(torch.int16))


def test_window_on_the_gqa_workload():
    dev = require_gpu()
    base = config_workload(4, seed=0, batch=8, block_size=16)
    for W in (256, 1000):
        w = _release_before_window(base, W)
        ref = oracle.paged_decode_window(w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.scale, W)
        note(f"GQA window W={W}")
        got, _ = _run(w, dev, W)
        assert_close(got, ref, "bf16", f"GQA window {W}")


@pytest.mark.parametrize("dtype,group,bs", [("bf16", 8, 16), ("f16", 1, 32)])
def test_window_long_contexts(dtype, group, bs):
    dev = require_gpu()
    lens = np.array([32769, 20000, 4097, 4096, 100, 4095], np.int32)
    base = build_paged(f"win-long-{dtype}", 410 + group, 1, lens, bs, 4, 4 * group, 128, dtype)
    w = _release_before_window(base, 4096)
    ref = oracle.paged_decode_window(w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.scale, 4096)
    for P in (0, 512, 4096):
        note(f"long window dtype={dtype} G={group} bs={bs} P={P}")
        got, _ = _run(w, dev, 4096, P)
        assert_close(got, ref, dtype, f"long window {dtype} G={group} P={P}")


def test_window_ignores_garbage_before_it_and_flags_bad_ids_inside():
    dev = require_gpu()
    lens = np.array([300, 64, 17], np.int32)
    base = build_paged("win-ids", 420, 0, lens, 16, 2, 2, 128, "f16")
    w = _release_before_window(base, 40)
    ref = oracle.paged_decode_window(w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.scale, 40)
    junk = w.block_table.copy()
    for b, L in enumerate(w.context_lens):
        n = max(0, int(L) - 40) // 16
        junk[b, :n] = 1 << 30  # out of the pool, but before the window: never read
    note("window with garbage ids before it")
    got, _ = _run(dataclasses.replace(w, block_table=junk), dev, 40, 32)
    assert_close(got, ref, "f16", "garbage before the window")
    bad = w.block_table.copy()
    bad[0, (300 - 1) // 16] = 1 << 30  # inside sequence 0's window
    t = dataclasses.replace(w, block_table=bad).to_device(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    note("window with a bad id inside it")
    out = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"], 300, w.scale,
                     partition_size=32, err_flag=err, window=40)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    o = out.float().cpu().numpy()
    assert np.all(np.isnan(o[0]))
    assert_close(o[1:].astype(np.float64), ref[1:], "f16", "other sequences after a bad id")
