"""GPU: every (sequence, head) row of the 32K-token beam step against the oracle.

The workload is 8 groups x 4 beams, 32 heads, head_dim 128, bf16, block_size 32, with a
30720-token prefix shared by the beams of a group ([BlockManager essay] §4.2; [KV Block
course] §3.4 on reference-counted blocks). The library runs the step once on the device:
copy-on-write of the last shared block (24 pairs), the fused append + decode at L = 32769
(default partitions, so the reduce pass writes the rows), then pa_decode at 512-token and
default partitions and pa_decode_beams at default and 512-token partitions over the grown
pools. A pristine device copy of the generator's pools, taken before the library touches
them, feeds the oracle one group at a time (copy-on-write, append and float64 decode of its
4 beams x 32 heads), and all five outputs are compared row by row.
"""

import concurrent.futures as cf
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_indexed_amd import ops
from tests.gpu_util import assert_close, note, require_gpu
from workloads.longctx import beam_workload, host_subset

pytestmark = pytest.mark.gpu

GROUPS = 8
BEAMS = 4


@pytest.fixture(scope="module")
def step_outputs():
    dev = require_gpu()
    note("config 5 full rows: building the 32K beam workload on the device")
    w = beam_workload(dev)
    t = w.tensors
    assert w.groups == GROUPS and w.beams == BEAMS
    # the generator's pools before the library runs: the oracle's only source of K/V
    pristine = dataclasses.replace(w, tensors=dict(t, k_pool=t["k_pool"].clone(), v_pool=t["v_pool"].clone()))
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    L = w.context
    outs = {}
    note("config 5 full rows: copy-on-write (24 pairs)")
    ops.copy_blocks(t["k_pool"], t["v_pool"], t["copy_pairs"], err_flag=err)
    note("config 5 full rows: fused append + decode, default partitions")
    outs["decode_append"] = ops.decode_append(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"],
                                              L + 1, w.scale, t["new_key"], t["new_value"], t["slot_mapping"],
                                              err_flag=err)
    for P in (512, 0):
        note(f"config 5 full rows: pa_decode at L + 1, P={P}")
        outs[f"decode P={P}"] = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"],
                                           L + 1, w.scale, partition_size=P, err_flag=err)
    for P in (0, 512):
        note(f"config 5 full rows: pa_decode_beams at L + 1, P={P}")
        outs[f"decode_beams P={P}"] = ops.decode_beams(t["q"], t["k_pool"], t["v_pool"], t["block_table"],
                                                       t["lens_after"], L + 1, w.scale, w.beams, partition_size=P,
                                                       err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    host_outs = {k: v.float().cpu().numpy().astype(np.float64) for k, v in outs.items()}
    del outs
    yield w, pristine, host_outs
    del pristine
    torch.cuda.empty_cache()


@pytest.mark.parametrize("group", range(GROUPS))
def test_config5_every_row(step_outputs, group):
    w, pristine, outs = step_outputs
    seqs = list(range(group * BEAMS, (group + 1) * BEAMS))
    heads = list(range(w.num_q_heads))
    note(f"config 5 full rows: oracle for group {group} (sequences {seqs[0]}-{seqs[-1]}, all heads)")
    host = host_subset(pristine, seqs, heads)
    k1, v1 = oracle.copy_blocks(host["k_pool"], host["v_pool"], host["copy_pairs"])
    k2, v2 = oracle.reshape_and_cache(k1, v1, host["new_key"], host["new_value"], host["slot_mapping"])
    del k1, v1
    lens = np.full(len(seqs), w.context + 1, np.int32)
    pairs = [(i, h) for i in range(len(seqs)) for h in heads]
    # one oracle call per (sequence, head), several at a time (numpy releases the GIL)
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        rows = list(ex.map(lambda p: oracle.paged_decode_heads(host["q"], k2, v2, host["table"], lens, w.scale,
                                                               [p])[0], pairs))
    ref = np.stack(rows).reshape(len(seqs), len(heads), -1)
    for name, o in outs.items():
        assert_close(o[seqs], ref, "bf16", f"config 5 group {group} all rows, {name}")
