"""pa_decode_append_noalloc (the fused step with the library's static scratch in place of a
workspace) against pa_decode_append with a caller workspace: outputs and pools bit for bit
(same kernels, same partitions, same records), on two calls in a row, the second smaller, and
the rejection of a call whose workspace would exceed the scratch (no launch)."""

import ctypes

import pytest
import torch

from paged_kv_cache_indexed_amd import _lib, ops
from tests.gpu_util import note, require_gpu
from workloads import config_workload

_INT = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def _bits(x):
    return x.view(_INT[x.dtype])


def _compare(w, dev, P):
    """One no-alloc call and one workspace call from identical device inputs."""
    ta, tb = w.to_device(dev), w.to_device(dev)
    L = int(w.lens_after_append.max())
    desc = _lib.CacheDesc.of(ta["k_pool"])
    assert _lib.pa_decode_workspace_bytes(desc, w.batch, w.num_q_heads, L, P) > 0, "the case must use a workspace"
    err_a = torch.zeros(1, dtype=torch.int32, device=dev)
    err_b = torch.zeros(1, dtype=torch.int32, device=dev)
    out_a = torch.full_like(ta["q"], float("nan"))
    _lib.pa_decode_append_noalloc(desc, out_a, ta["q"], ta["k_pool"], ta["v_pool"], ta["block_table"],
                                  ta["lens_after"], L, w.scale, ta["new_key"], ta["new_value"], ta["slot_mapping"],
                                  P, err_a)
    out_b = ops.decode_append(tb["q"], tb["k_pool"], tb["v_pool"], tb["block_table"], tb["lens_after"], L, w.scale,
                              tb["new_key"], tb["new_value"], tb["slot_mapping"], partition_size=P, err_flag=err_b)
    torch.cuda.synchronize()
    assert int(err_a.item()) == 0 and int(err_b.item()) == 0
    assert torch.equal(_bits(out_a), _bits(out_b)), "no-alloc output differs from the workspace call"
    for a, b in ((ta["k_pool"], tb["k_pool"]), (ta["v_pool"], tb["v_pool"])):
        assert torch.equal(_bits(a), _bits(b)), "no-alloc append wrote a different pool"


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice():
    dev = require_gpu()
    # first call: 64 long-tail sequences split into 64-token partitions (reduce pass, rows
    # written by it); second call: a smaller batch and shorter partitions on the same scratch
    for kw, P in ((dict(batch=64, heads=8), 64), (dict(batch=12, heads=4), 32)):
        w = config_workload(3, seed=21, **kw)
        note(f"noalloc vs workspace decode_append cfg 3 {kw} P={P}")
        _compare(w, dev, P)
    # a grouped-query case on the matrix-core path, smaller again
    w = config_workload(4, seed=22, batch=2)
    note("noalloc vs workspace decode_append cfg 4 batch 2 P=512")
    _compare(w, dev, 512)


def test_noalloc_rejects_more_than_its_scratch():
    """Argument checks run on the host before any device call (no GPU needed)."""
    lib = _lib.load()
    desc = _lib.CacheDesc(100000, 16, 32, 128, _lib.PA_F16).c()
    batch, heads, L, P = 1024, 32, 16384, 256
    need = _lib.pa_decode_workspace_bytes(_lib.CacheDesc(100000, 16, 32, 128, _lib.PA_F16), batch, heads, L, P)
    assert need > _lib.PA_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the call returns before launching
    st = lib.pa_decode_append_noalloc(ctypes.byref(desc), fake, fake, fake, fake, fake, 1024, fake, batch, heads, L,
                                      1.0, fake, fake, fake, P, None, None)
    assert st == _lib.PA_ERR_SCRATCH_LIMIT
    assert "SCRATCH" in _lib.pa_status_string(st)
    # batch 0 is a no-op, as for pa_decode_append
    st = lib.pa_decode_append_noalloc(ctypes.byref(desc), None, None, None, None, None, 4, None, 0, 32, 10, 1.0,
                                      None, None, None, 0, None, None)
    assert st == _lib.PA_OK
