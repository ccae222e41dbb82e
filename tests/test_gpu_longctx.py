"""GPU: the 32K-token beam workload with shared-prefix blocks, copy-on-write and append.

8 groups x 4 beams, 32 heads, head_dim 128, bf16, block_size 32; the first 30720 tokens of
each group are one set of physical blocks shared by its 4 beams. The step copies the last
shared block for beams 1-3 (24 pairs), appends one token per beam and decodes at L = 32769
over 512-token partitions with the log-sum-exp reduce.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_indexed_amd import ops
from tests.gpu_util import assert_close, note, require_gpu
from workloads.longctx import beam_workload, host_subset

pytestmark = pytest.mark.gpu

SEQS = [0, 1, 2, 3, 21]   # all beams of group 0, one beam of group 5
HEADS = [0, 13, 31]


def test_config5_copy_on_write_append_decode():
    dev = require_gpu()
    note("config 5: building the 32K beam workload on the device")
    w = beam_workload(dev)
    t = w.tensors
    assert w.unique_blocks == 9728 and w.copy_pairs.shape == (24, 2)
    host = host_subset(w, SEQS, HEADS)  # snapshot before the library touches anything
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    L = w.context

    note("config 5: decode with shared prefix blocks, P=512")
    out0 = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table_shared"], t["context_lens"], L,
                      w.scale, partition_size=512, err_flag=err)
    note("config 5: copy-on-write of the last shared block (24 pairs)")
    ops.copy_blocks(t["k_pool"], t["v_pool"], t["copy_pairs"], err_flag=err)
    torch.cuda.synchronize()
    src = torch.from_numpy(w.copy_pairs[:, 0].astype(np.int64)).to(dev)
    dst = torch.from_numpy(w.copy_pairs[:, 1].astype(np.int64)).to(dev)
    for pool in (t["k_pool"], t["v_pool"]):
        assert torch.equal(pool[src].view(torch.int16), pool[dst].view(torch.int16)), "copy not bit-exact"

    note("config 5: decode with the private copies is bitwise unchanged")
    out1 = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"], L, w.scale,
                      partition_size=512, err_flag=err)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))

    note("config 5: append one token per beam")
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], t["slot_mapping"],
                          err_flag=err)
    torch.cuda.synchronize()
    blk = torch.from_numpy(w.slot_mapping // w.block_size).long().to(dev)
    off = torch.from_numpy(w.slot_mapping % w.block_size).long().to(dev)
    got_k = t["k_pool"][blk, :, off, :]
    assert torch.equal(got_k.view(torch.int16), t["new_key"].view(torch.int16))

    outs = {}
    for P in (512, 0):
        note(f"config 5: decode at L={L + 1}, P={P}")
        outs[P] = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"], L + 1,
                             w.scale, partition_size=P, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for P, o in outs.items():
        assert torch.isfinite(o.float()).all(), f"non-finite output P={P}"

    note("config 5: oracle on the sampled sequences and heads")
    k1, v1 = oracle.copy_blocks(host["k_pool"], host["v_pool"], host["copy_pairs"])
    k2, v2 = oracle.reshape_and_cache(k1, v1, host["new_key"], host["new_value"], host["slot_mapping"])
    pairs = [(i, j) for i in range(len(SEQS)) for j in range(len(HEADS))]
    lens = np.full(len(SEQS), L + 1, np.int32)
    ref = oracle.paged_decode_heads(host["q"], k2, v2, host["table"], lens, w.scale, pairs)
    for P, o in outs.items():
        got = o.float().cpu().numpy()[np.ix_(SEQS, HEADS)].reshape(len(pairs), -1).astype(np.float64)
        assert_close(got, ref, "bf16", f"config 5 sampled outputs P={P}")

    # the library's pool bytes equal the oracle's after copy-on-write and append
    ids = torch.from_numpy(host["block_ids"]).to(dev)
    hs = torch.tensor(HEADS, device=dev)
    gk = t["k_pool"].index_select(0, ids).index_select(1, hs).float().cpu().numpy()
    gv = t["v_pool"].index_select(0, ids).index_select(1, hs).float().cpu().numpy()
    assert np.array_equal(gk, k2, equal_nan=True) and np.array_equal(gv, v2, equal_nan=True)


def test_config5_fused_step():
    """The benchmark's config 5 step: copy-on-write, then the append fused into the decode
    (default partitions, so the reduce pass writes the rows), on sampled outputs."""
    dev = require_gpu()
    note("config 5 fused: building the 32K beam workload on the device")
    w = beam_workload(dev)
    t = w.tensors
    host = host_subset(w, SEQS, HEADS)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    L = w.context
    ops.copy_blocks(t["k_pool"], t["v_pool"], t["copy_pairs"], err_flag=err)
    note("config 5 fused: decode_append at L + 1")
    out = ops.decode_append(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"], L + 1, w.scale,
                            t["new_key"], t["new_value"], t["slot_mapping"], err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    blk = torch.from_numpy(w.slot_mapping // w.block_size).long().to(dev)
    off = torch.from_numpy(w.slot_mapping % w.block_size).long().to(dev)
    for pool, new in ((t["k_pool"], t["new_key"]), (t["v_pool"], t["new_value"])):
        assert torch.equal(pool[blk, :, off, :].view(torch.int16), new.view(torch.int16)), "appended rows differ"
    k1, v1 = oracle.copy_blocks(host["k_pool"], host["v_pool"], host["copy_pairs"])
    k2, v2 = oracle.reshape_and_cache(k1, v1, host["new_key"], host["new_value"], host["slot_mapping"])
    pairs = [(i, j) for i in range(len(SEQS)) for j in range(len(HEADS))]
    ref = oracle.paged_decode_heads(host["q"], k2, v2, host["table"], np.full(len(SEQS), L + 1, np.int32), w.scale,
                                    pairs)
    got = out.float().cpu().numpy()[np.ix_(SEQS, HEADS)].reshape(len(pairs), -1).astype(np.float64)
    assert_close(got, ref, "bf16", "config 5 fused sampled outputs")


def test_config5_beam_decode_step():
    """The benchmark's config 5 step with --beams 4: copy-on-write, append, then pa_decode_beams
    (the shared prefix read once per group of 4 beams; the copied last shared block and the
    tails per beam), on sampled outputs, for the default and the 512-token partitions."""
    dev = require_gpu()
    note("config 5 beams: building the 32K beam workload on the device")
    w = beam_workload(dev)
    t = w.tensors
    host = host_subset(w, SEQS, HEADS)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    L = w.context
    ops.copy_blocks(t["k_pool"], t["v_pool"], t["copy_pairs"], err_flag=err)
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_pool"], t["v_pool"], t["slot_mapping"], err_flag=err)
    k1, v1 = oracle.copy_blocks(host["k_pool"], host["v_pool"], host["copy_pairs"])
    k2, v2 = oracle.reshape_and_cache(k1, v1, host["new_key"], host["new_value"], host["slot_mapping"])
    pairs = [(i, j) for i in range(len(SEQS)) for j in range(len(HEADS))]
    ref = oracle.paged_decode_heads(host["q"], k2, v2, host["table"], np.full(len(SEQS), L + 1, np.int32), w.scale,
                                    pairs)
    for P in (0, 512):
        note(f"config 5 beams: decode_beams at L + 1, P={P}")
        out = ops.decode_beams(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"], L + 1, w.scale,
                               w.beams, partition_size=P, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.isfinite(out.float()).all()
        got = out.float().cpu().numpy()[np.ix_(SEQS, HEADS)].reshape(len(pairs), -1).astype(np.float64)
        assert_close(got, ref, "bf16", f"config 5 beam decode sampled outputs P={P}")
