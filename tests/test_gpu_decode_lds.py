"""GPU: the grouped-query decode on its LDS path (fp16/bf16 pools, head_dim 128, 4 or 8 query
heads per kv head: tiles reach LDS through direct buffer loads, and the P V operand comes
from transpose reads) against the float64 oracle.

Partition sizes from 64 tokens to whole sequences: short partitions in grids of 1024 or more
work-groups run the 4-wave form, the rest the 8-wave form. Unused pool slots hold NaN, so a
read of padding would show. (The other decode tests at head_dim 128 with 4 or 8 heads per kv
head run on this path too.)
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_indexed_amd import ops
from paged_kv_cache_indexed_amd._lib import (PA_FLAG_BAD_BLOCK_ID, PA_FLAG_BAD_LENGTH, PA_FLAG_EMPTY_CONTEXT,
                                             CacheDesc, pa_decode_partition_size)
from tests.gpu_util import assert_close, gpu_decode, note, oracle_decode, require_gpu
from workloads import build_paged

pytestmark = pytest.mark.gpu

# short and long sequences in one batch: tiles that start past the length, a last tile with
# one token, lengths one past and one short of a tile and of a partition
_LENS = np.array([1, 15, 16, 17, 300, 1151, 1152, 1153, 2049, 2500, 3000, 4100], np.int32)


@pytest.mark.parametrize("dtype,group,bs", [("bf16", 8, 16), ("f16", 8, 16), ("bf16", 4, 16), ("f16", 4, 32),
                                            ("bf16", 8, 64), ("bf16", 8, 256), ("f16", 8, 512), ("bf16", 8, 8),
                                            ("f16", 4, 8)])
def test_lds_path_matches_oracle(dtype, group, bs):
    dev = require_gpu()
    w = build_paged(f"lds-{dtype}-{group}-{bs}", 500 + group, bs, _LENS, bs, 2, 2 * group, 128, dtype)
    ref = oracle_decode(w)
    t = w.to_device(dev)
    whole = -(-int(_LENS.max()) // bs) * bs
    # 64 and 128: 1560 and 792 work-groups of 2 kv heads x 12 sequences (4- and 8-wave forms)
    for P in sorted({max(64, bs), max(128, bs), 1152 if bs <= 128 else 1536, 2048, 4096, whole}):
        note(f"lds path dtype={dtype} G={group} bs={bs} P={P}")
        got, _ = gpu_decode(w, dev, partition_size=P, tensors=t)
        assert_close(got, ref, dtype, f"lds path {dtype} G={group} bs={bs} P={P}")


def test_lds_path_one_partition_per_sequence_at_full_size():
    """B = 32 sequences of 2049 tokens, 8 kv heads of 8 query heads (the grouped-query
    workload's shape; here with ragged lengths below it), one partition each."""
    dev = require_gpu()
    rng = np.random.default_rng(5)
    lens = rng.integers(1200, 2050, 32).astype(np.int32)
    lens[0] = 2049
    w = build_paged("lds-full", 510, 16, lens, 16, 8, 64, 128, "bf16")
    ref = oracle_decode(w)
    t = w.to_device(dev)
    assert pa_decode_partition_size(CacheDesc.of(t["k_pool"]), 32, 64, 2049, 0) == 2064
    note("lds path B=32 ragged up to 2049")
    got, _ = gpu_decode(w, dev)
    assert_close(got, ref, "bf16", "lds path B=32 ragged up to 2049")


def _release_before_window(w, window):
    tab = w.block_table.copy()
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    for b, L in enumerate(w.context_lens):
        n = max(0, int(L) - window) // w.block_size
        ids = tab[b, :n]
        kp[ids] = np.nan
        vp[ids] = np.nan
        tab[b, :n] = -1
    return dataclasses.replace(w, block_table=tab, k_pool=kp, v_pool=vp)


@pytest.mark.parametrize("window", [1200, 2000, 4100])
def test_lds_path_sliding_window(window):
    """A window starting inside a tile and inside a block, blocks before it released (-1 ids,
    NaN contents)."""
    dev = require_gpu()
    base = build_paged("lds-window", 520, 16, _LENS, 16, 2, 16, 128, "bf16")
    w = _release_before_window(base, window)
    ref = oracle.paged_decode_window(w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.scale, window)
    t = w.to_device(dev)
    for P in (64, 1152, 2048):
        note(f"lds path window={window} P={P}")
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        out = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"], int(_LENS.max()),
                         w.scale, partition_size=P, err_flag=err, window=window)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert_close(out.float().cpu().numpy().astype(np.float64), ref, "bf16", f"lds window={window} P={P}")


@pytest.mark.parametrize("P", [64, 1152, 2048, 4112])
def test_lds_path_fused_append(P):
    """pa_decode_append: the new token's rows replace their slot in the staged tile. Outputs
    bit for bit those of the separate append and decode, pools bit for bit, and the oracle."""
    dev = require_gpu()
    w = build_paged("lds-append", 530, 16, _LENS, 16, 2, 16, 128, "bf16")
    t1, t2 = w.to_device(dev), w.to_device(dev)
    L = int(w.lens_after_append.max())
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    note(f"lds path fused append P={P}")
    fused = ops.decode_append(t1["q"], t1["k_pool"], t1["v_pool"], t1["block_table"], t1["lens_after"], L, w.scale,
                              t1["new_key"], t1["new_value"], t1["slot_mapping"], partition_size=P, err_flag=err)
    ops.reshape_and_cache(t2["new_key"], t2["new_value"], t2["k_pool"], t2["v_pool"], t2["slot_mapping"])
    sep = ops.decode(t2["q"], t2["k_pool"], t2["v_pool"], t2["block_table"], t2["lens_after"], L, w.scale,
                     partition_size=P)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(t1["k_pool"].view(torch.int16), t2["k_pool"].view(torch.int16))
    assert torch.equal(t1["v_pool"].view(torch.int16), t2["v_pool"].view(torch.int16))
    assert torch.equal(fused.view(torch.int16), sep.view(torch.int16))
    ka, va = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    ref = oracle.paged_decode(w.q, ka, va, w.block_table, w.lens_after_append, w.scale)
    assert_close(fused.float().cpu().numpy(), ref, "bf16", f"lds fused append P={P}")


def test_lds_path_bad_inputs():
    """A bad block id poisons only its sequence (NaN outputs, flag); an empty context and a
    length past max_context_len are flagged and give NaN rows; the others are exact."""
    dev = require_gpu()
    lens = _LENS.copy()
    w = build_paged("lds-bad", 540, 16, lens, 16, 2, 16, 128, "f16")
    tab = w.block_table.copy()
    tab[10, 100] = w.k_pool.shape[0] + 5  # sequence 10 (3000 tokens): an id past the pool
    ref = oracle_decode(w)
    t = w.to_device(dev)
    t["block_table"] = torch.from_numpy(tab).to(dev)
    ml = tab.shape[1] * 16  # the table's capacity, the longest max_context_len it allows
    bad_lens = torch.from_numpy(lens.copy()).to(dev)
    bad_lens[0] = 0
    bad_lens[1] = ml + 1  # past max_context_len
    for P in (64, 1152, 2048):
        note(f"lds path bad inputs P={P}")
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        out = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], bad_lens, ml, w.scale,
                         partition_size=P, err_flag=err)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert int(err.item()) == PA_FLAG_BAD_BLOCK_ID | PA_FLAG_EMPTY_CONTEXT | PA_FLAG_BAD_LENGTH
        assert np.isnan(got[[0, 1, 10]]).all()
        keep = [i for i in range(len(lens)) if i not in (0, 1, 10)]
        assert_close(got[keep], ref[keep], "f16", f"lds path next to bad inputs P={P}")
