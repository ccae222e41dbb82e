"""The measurement entry points (include/pagedkv_measure.h): argument checks on the CPU (they
return before any device call), and one launch of each on the GPU."""

import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_indexed_amd import _lib
from tests.gpu_util import note, require_gpu
from workloads import config_workload


def _raw_gather(desc, k=None, v=None, table=None, mbs=1, lens=None, batch=1, max_len=1, sink=None):
    c = desc.c()
    return _lib.load().pa_measure_gather_read(ctypes.byref(c), k, v, table, mbs, lens, batch, max_len, sink, None)


def test_gather_read_rejects_bad_arguments():
    ok16 = _lib.CacheDesc(100, 16, 4, 128, _lib.PA_F16)
    fake = ctypes.c_void_p(4096)  # never dereferenced: every case returns before a launch
    # rows of 64 bytes in 8-token blocks hold 512 bytes per kv head: a wave load would cross a block
    assert _raw_gather(_lib.CacheDesc(100, 8, 4, 64, _lib.PA_FP8_E4M3), fake, fake, fake, 1, fake, 1, 1,
                       fake) == _lib.PA_ERR_UNSUPPORTED
    assert _raw_gather(ok16, None, fake, fake, 1, fake, 1, 1, fake) == _lib.PA_ERR_INVALID_ARGUMENT
    assert _raw_gather(ok16, fake, fake, fake, 1, fake, 1, 1, None) == _lib.PA_ERR_INVALID_ARGUMENT
    assert _raw_gather(ok16, fake, fake, fake, 0, fake, 1, 1, fake) == _lib.PA_ERR_INVALID_ARGUMENT
    assert _raw_gather(ok16, fake, fake, fake, 1, fake, -1, 1, fake) == _lib.PA_ERR_INVALID_ARGUMENT
    assert _raw_gather(ok16, ctypes.c_void_p(4104), fake, fake, 1, fake, 1, 1, fake) == _lib.PA_ERR_INVALID_ARGUMENT
    assert _raw_gather(ok16, fake, fake, fake, 1, fake, 0, 1, fake) == _lib.PA_OK  # empty batch: nothing to do


@pytest.mark.gpu
def test_gather_read_runs_on_a_paged_cache():
    dev = require_gpu()
    w = config_workload(2, seed=1, batch=16, heads=8)
    t = w.to_device(dev)
    sink = torch.zeros(w.batch * w.num_kv_heads, dtype=torch.float32, device=dev)
    note("gather read, config 2 shape")
    desc = _lib.CacheDesc.of(t["k_pool"])
    for _ in range(3):
        _lib.pa_measure_gather_read(desc, t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"],
                                    int(w.lens_after_append.max()), sink)
    torch.cuda.synchronize()
    # the sink is written only when a work-group's XOR of what it read hits one fixed value
    assert int((sink != 0).sum().item()) <= 1
    # lengths past max_context_len, and ids outside the pool, are skipped rather than read
    bad = t["block_table"].clone()
    bad[0, 0] = w.num_blocks + 5
    _lib.pa_measure_gather_read(desc, t["k_pool"], t["v_pool"], bad, t["lens_after"], 8, sink)
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_stream_read_runs():
    dev = require_gpu()
    buf = torch.zeros(1 << 22, dtype=torch.float32, device=dev)
    sink = torch.zeros(64, dtype=torch.float32, device=dev)
    note("stream read, 16 MiB")
    _lib.pa_measure_stream_read(buf, sink, 64)
    torch.cuda.synchronize()
    assert int((sink != 0).sum().item()) == 0  # an all-zero buffer XORs to 0, never the trigger value
    with pytest.raises(_lib.PagedKVError):
        _lib.pa_measure_stream_read(buf[1:], sink, 64)  # 4 bytes off the 16-byte alignment
