"""GPU: pa_reshape_and_cache and pa_copy_blocks are bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_indexed_amd import ops
from paged_kv_cache_indexed_amd._lib import PA_FLAG_BAD_COPY_PAIR, PA_FLAG_BAD_SLOT
from tests.gpu_util import note, require_gpu
from workloads import build_paged

pytestmark = pytest.mark.gpu

_TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_IV = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}


def _bits_cpu(x_f32: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(_TD[dtype]).view(_IV[dtype])


def _bits_dev(t: torch.Tensor, dtype: str) -> torch.Tensor:
    return t.cpu().view(_IV[dtype])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("bs", [8, 16, 64])
def test_reshape_and_cache_bit_exact(dtype, head_dim, bs):
    dev = require_gpu()
    note(f"reshape_and_cache dtype={dtype} d={head_dim} bs={bs}")
    lens = np.array([0, 5, bs - 1, bs, 3 * bs + 2, 40], np.int32)
    w = build_paged("cache", 90, 1, lens, bs, 3, 3, head_dim, dtype)
    t = w.to_device(dev)
    slots = w.slot_mapping.copy()
    slots[2] = -1  # a padding token is never written
    slots_t = torch.from_numpy(slots).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], slots_t, err_flag=err)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, slots)
    assert torch.equal(_bits_dev(t["k_pool"], dtype), _bits_cpu(ek, dtype))
    assert torch.equal(_bits_dev(t["v_pool"], dtype), _bits_cpu(ev, dtype))
    assert int(err.item()) == 0


def test_reshape_and_cache_bad_slot_and_empty():
    dev = require_gpu()
    note("reshape_and_cache bad slot / empty")
    w = build_paged("cache", 91, 2, np.array([3, 9], np.int32), 8, 2, 2, 128, "f16")
    t = w.to_device(dev)
    before_k = t["k_pool"].clone()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    bad = torch.tensor([w.num_blocks * 8, -3], dtype=torch.int32, device=dev)
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], bad, err_flag=err)
    ops.reshape_and_cache(t["new_key"][:0], t["new_value"][:0], t["k_pool"], t["v_pool"], bad[:0])
    torch.cuda.synchronize()
    assert int(err.item()) == PA_FLAG_BAD_SLOT
    assert torch.equal(before_k.view(torch.int16), t["k_pool"].view(torch.int16))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_copy_blocks_bit_exact(dtype):
    dev = require_gpu()
    note(f"copy_blocks dtype={dtype}")
    w = build_paged("cow", 92, 3, np.array([40, 17, 64], np.int32), 16, 4, 8, 128, dtype, spare=0.5)
    t = w.to_device(dev)
    used = set(w.block_table[w.block_table >= 0].tolist())
    free = [i for i in range(w.num_blocks) if i not in used]
    pairs = np.array([[w.block_table[0, 0], free[0]], [w.block_table[1, 1], free[1]],
                      [w.block_table[2, 3], free[2]]], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ops.copy_blocks(t["k_pool"], t["v_pool"], torch.from_numpy(pairs).to(dev), err_flag=err)
    torch.cuda.synchronize()
    ek, ev = oracle.copy_blocks(w.k_pool, w.v_pool, pairs)
    assert torch.equal(_bits_dev(t["k_pool"], dtype), _bits_cpu(ek, dtype))
    assert torch.equal(_bits_dev(t["v_pool"], dtype), _bits_cpu(ev, dtype))
    assert int(err.item()) == 0


def test_copy_blocks_bad_pairs_flagged():
    dev = require_gpu()
    note("copy_blocks bad pairs")
    w = build_paged("cow", 93, 4, np.array([20], np.int32), 16, 2, 2, 64, "bf16", spare=2.0)
    t = w.to_device(dev)
    nb = w.num_blocks
    before = t["k_pool"].clone()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    bad = torch.tensor([[0, 0], [-1, 1], [1, nb]], dtype=torch.int32, device=dev)
    ops.copy_blocks(t["k_pool"], t["v_pool"], bad, err_flag=err)
    ops.copy_blocks(t["k_pool"], t["v_pool"], bad[:0])
    torch.cuda.synchronize()
    assert int(err.item()) == PA_FLAG_BAD_COPY_PAIR
    assert torch.equal(before.view(torch.int16), t["k_pool"].view(torch.int16))
