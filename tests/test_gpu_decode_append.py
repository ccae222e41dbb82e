"""GPU: the fused append + decode (pa_decode_append) against the two separate calls (pools
bit for bit; outputs bit for bit on the matrix cores, within tolerance on the VALU kernels,
where the new token is summed in another order) and against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_cache as o8
from paged_kv_cache_indexed_amd import ops
from tests.gpu_util import assert_close, note, require_gpu
from workloads import build_paged, config_workload

pytestmark = pytest.mark.gpu

_INT = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def _both(w, dev, P=0, slots=None):
    """Fused and separate runs from identical device inputs; returns (fused, separate,
    err_fused, pools_fused, pools_separate)."""
    t1, t2 = w.to_device(dev), w.to_device(dev)
    sl = t1["slot_mapping"] if slots is None else torch.as_tensor(slots, dtype=torch.int32, device=dev)
    L = int(w.lens_after_append.max())
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    fused = ops.decode_append(t1["q"], t1["k_pool"], t1["v_pool"], t1["block_table"], t1["lens_after"], L, w.scale,
                              t1["new_key"], t1["new_value"], sl, partition_size=P, err_flag=err)
    ops.reshape_and_cache(t2["new_key"], t2["new_value"], t2["k_pool"], t2["v_pool"], sl)
    sep = ops.decode(t2["q"], t2["k_pool"], t2["v_pool"], t2["block_table"], t2["lens_after"], L, w.scale,
                     partition_size=P)
    torch.cuda.synchronize()
    return fused, sep, int(err.item()), (t1["k_pool"], t1["v_pool"]), (t2["k_pool"], t2["v_pool"])


def _bits(x):
    return x.view(_INT[x.dtype])


@pytest.mark.parametrize("cfg,kw,P", [(1, {}, 0), (1, {}, 32), (2, dict(batch=16, heads=8), 0),
                                      (2, dict(batch=16, heads=8), 64), (2, dict(batch=16, heads=8), 256),
                                      (3, dict(batch=64, heads=4), 0), (4, dict(batch=8), 0), (4, dict(batch=8), 512),
                                      (3, dict(batch=64, heads=4, block_size=8), 0),
                                      (4, dict(batch=8, block_size=8), 0), (4, dict(batch=8, block_size=8), 24),
                                      (4, dict(batch=8), 1152), (4, dict(batch=8, block_size=256), 2304)])
def test_fused_equals_separate_calls_bitwise(cfg, kw, P):
    dev = require_gpu()
    w = config_workload(cfg, seed=11, **kw)
    note(f"decode_append cfg={cfg} {kw} P={P}")
    fused, sep, err, pf, ps = _both(w, dev, P)
    assert err == 0
    for a, b in zip(pf, ps):
        assert torch.equal(_bits(a), _bits(b)), "fused append wrote a different pool"
    if cfg == 4:  # matrix cores: the new row takes its usual place in the stream, bit for bit
        assert torch.equal(_bits(fused), _bits(sep)), "fused output differs from the separate calls"
    else:  # VALU: the new token joins one row stream after the loop (another summation order)
        assert_close(fused.float().cpu().numpy(), sep.float().cpu().numpy().astype(np.float64), w.dtype,
                     f"fused vs separate cfg {cfg} P={P}")
    ka, va = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    ref = oracle.paged_decode(w.q, ka, va, w.block_table, w.lens_after_append, w.scale)
    assert_close(fused.float().cpu().numpy(), ref, w.dtype, f"decode_append cfg {cfg} P={P}")


@pytest.mark.parametrize("P", [0, 64])
def test_fused_skips_negative_slots_and_flags_wrong_ones(P):
    """P = 64 splits every context, so the rows are written by the reduce pass."""
    dev = require_gpu()
    w = config_workload(2, seed=12, batch=8, heads=4)
    slots = w.slot_mapping.copy()
    slots[1] = -1                       # no append: the decode reads the old (NaN) slot
    slots[2] = slots[3]                 # not this sequence's last position: flagged, not written
    note(f"decode_append slots P={P}")
    fused, sep, err, pf, ps = _both(w, dev, P, slots)
    assert err & 8
    o = fused.float().cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))  # their last rows were never written
    keep = [0] + list(range(3, 8))
    ka, va = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key[keep], w.new_value[keep], w.slot_mapping[keep])
    ref = oracle.paged_decode(w.q, ka, va, w.block_table, w.lens_after_append, w.scale)
    assert_close(o[keep], ref[keep], "f16", "decode_append next to skipped and bad slots")
    for got, want in zip(pf, (ka, va)):  # only the kept sequences' slots were written
        g = got.float().cpu().numpy()
        assert np.array_equal(np.isnan(g), np.isnan(want)) and np.array_equal(np.nan_to_num(g), np.nan_to_num(want))


@pytest.mark.parametrize("P", [0, 64])
def test_fused_poisoned_sequences(P):
    """Bad block ids and an empty context next to valid sequences: NaN outputs for the
    poisoned ones, exact outputs and appends for the others, and no row written through a
    bad id or for a bad length."""
    dev = require_gpu()
    w = config_workload(2, seed=14, batch=8, heads=4)
    bs = w.block_size
    L = w.lens_after_append.copy()
    table = w.block_table.copy()
    table[3, (L[3] - 1) // bs] = w.k_pool.shape[0] + 5  # the new token's block
    table[4, 0] = -7                                     # the first block only
    lens = L.copy()
    lens[5] = 0
    t = w.to_device(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    note(f"decode_append poisoned sequences P={P}")
    out = ops.decode_append(t["q"], t["k_pool"], t["v_pool"], torch.from_numpy(table).to(dev),
                            torch.from_numpy(lens).to(dev), int(L.max()), w.scale, t["new_key"], t["new_value"],
                            t["slot_mapping"], partition_size=P, err_flag=err)
    torch.cuda.synchronize()
    e = int(err.item())
    assert e & 1 and e & 4 and not e & 8
    o = out.float().cpu().numpy()
    assert all(np.all(np.isnan(o[b])) for b in (3, 4, 5))
    keep = [0, 1, 2, 6, 7]
    ka, va = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key[keep], w.new_value[keep], w.slot_mapping[keep])
    ref = oracle.paged_decode(w.q, ka, va, w.block_table, L, w.scale)
    assert_close(o[keep], ref[keep], "f16", f"valid sequences next to poisoned ones, P={P}")
    # sequence 4's last partition is valid when P splits its context: its row may land there
    s4 = int(w.slot_mapping[4])
    blk, off = s4 // bs, s4 % bs
    for got, want, new in zip((t["k_pool"], t["v_pool"]), (ka, va), (w.new_key, w.new_value)):
        g = got.float().cpu().numpy()
        row = g[blk, :, off].copy()
        assert np.array_equal(np.nan_to_num(row), np.nan_to_num(want[blk, :, off])) or \
            np.array_equal(row, new[4].astype(np.float16).astype(np.float32))
        g[blk, :, off] = want[blk, :, off]
        assert np.array_equal(np.isnan(g), np.isnan(want)) and np.array_equal(np.nan_to_num(g), np.nan_to_num(want))


def test_fused_on_a_multilayer_view():
    dev = require_gpu()
    w = config_workload(2, seed=13, batch=8, heads=4)
    t = w.to_device(dev)
    nb, hkv, bs, d = t["k_pool"].shape
    cache = torch.zeros((nb, 2, 3, hkv, bs, d), dtype=torch.float16, device=dev)
    cache[:, 0, 1].copy_(t["k_pool"])
    cache[:, 1, 1].copy_(t["v_pool"])
    L = int(w.lens_after_append.max())
    note("decode_append on a strided layer view")
    out = ops.decode_append(t["q"], cache[:, 0, 1], cache[:, 1, 1], t["block_table"], t["lens_after"], L, w.scale,
                            t["new_key"], t["new_value"], t["slot_mapping"])
    torch.cuda.synchronize()
    ka, va = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    ref = oracle.paged_decode(w.q, ka, va, w.block_table, w.lens_after_append, w.scale)
    assert_close(out.float().cpu().numpy(), ref, "f16", "decode_append multilayer")
    assert torch.all(cache[:, :, 0] == 0) and torch.all(cache[:, :, 2] == 0), "other layers were written"


# ---- 8-bit pools: pa_decode_append_fp8 against pa_reshape_and_cache_fp8 + pa_decode_fp8 -----

def _fp8_cache(w, dev):
    """Device (k codes, v codes, k scales, v scales) of the workload's context, quantised by the
    oracle's encoder; unwritten rows hold NaN codes and NaN scales."""
    dead = np.isnan(w.k_pool).any(-1)
    kc, ks = o8.quantize_rows(np.nan_to_num(w.k_pool))
    vc, vs = o8.quantize_rows(np.nan_to_num(w.v_pool))
    kc[dead], vc[dead] = o8.E4M3_NAN_CODE, o8.E4M3_NAN_CODE
    ks[dead], vs[dead] = np.nan, np.nan
    return [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (kc, vc, ks, vs)]


def _both_fp8(w, dev, P=0, slots=None):
    t = w.to_device(dev)
    c1, c2 = _fp8_cache(w, dev), _fp8_cache(w, dev)
    sl = t["slot_mapping"] if slots is None else torch.as_tensor(slots, dtype=torch.int32, device=dev)
    L = int(w.lens_after_append.max())
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    fused = ops.decode_append_fp8(t["q"], *c1, t["block_table"], t["lens_after"], L, w.scale, t["new_key"],
                                  t["new_value"], sl, partition_size=P, err_flag=err)
    ops.reshape_and_cache_fp8(t["new_key"], t["new_value"], *c2, sl)
    sep = ops.decode_fp8(t["q"], *c2, t["block_table"], t["lens_after"], L, w.scale, partition_size=P)
    torch.cuda.synchronize()
    return fused, sep, int(err.item()), c1, c2


def _same_bits(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


@pytest.mark.parametrize("cfg,kw,P", [(2, dict(batch=16, heads=8), 0), (2, dict(batch=16, heads=8), 64),
                                      (2, dict(batch=16, heads=8), 256), (3, dict(batch=64, heads=4), 0),
                                      (4, dict(batch=8), 0), (4, dict(batch=8), 512)])
def test_fused_fp8_equals_separate_calls(cfg, kw, P):
    """Codes and scales bit for bit; outputs bit for bit on the matrix cores (config 4) and
    within tolerance on the VALU kernels; and against the oracle's quantised append + decode."""
    dev = require_gpu()
    w = config_workload(cfg, seed=15, **kw)
    note(f"decode_append_fp8 cfg={cfg} {kw} P={P}")
    fused, sep, err, c1, c2 = _both_fp8(w, dev, P)
    assert err == 0
    for a, b in zip(c1, c2):
        assert _same_bits(a, b), "fused fp8 append wrote different codes or scales"
    if cfg == 4:
        assert torch.equal(_bits(fused), _bits(sep)), "fused fp8 output differs from the separate calls"
    else:
        assert_close(fused.float().cpu().numpy(), sep.float().cpu().numpy().astype(np.float64), w.dtype,
                     f"fused fp8 vs separate cfg {cfg} P={P}")
    kc, vc, ks, vs = (x.cpu().numpy() for x in _fp8_cache(w, torch.device("cpu")))
    kc, vc, ks, vs = o8.reshape_and_cache_fp8(kc, vc, ks, vs, w.new_key, w.new_value, w.slot_mapping)
    ref = o8.paged_decode_fp8(w.q, kc, vc, ks, vs, w.block_table, w.lens_after_append, w.scale)
    assert_close(fused.float().cpu().numpy(), ref, w.dtype, f"decode_append_fp8 cfg {cfg} P={P}")


def test_fused_fp8_slots():
    dev = require_gpu()
    w = config_workload(2, seed=16, batch=8, heads=4)
    slots = w.slot_mapping.copy()
    slots[1] = -1
    slots[2] = slots[3]
    note("decode_append_fp8 slots")
    fused, sep, err, c1, c2 = _both_fp8(w, dev, 0, slots)
    assert err & 8
    o = fused.float().cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    keep = [0] + list(range(3, 8))
    kc, vc, ks, vs = (x.cpu().numpy() for x in _fp8_cache(w, torch.device("cpu")))
    kc, vc, ks, vs = o8.reshape_and_cache_fp8(kc, vc, ks, vs, w.new_key[keep], w.new_value[keep],
                                              w.slot_mapping[keep])
    ref = o8.paged_decode_fp8(w.q, kc, vc, ks, vs, w.block_table, w.lens_after_append, w.scale)
    assert_close(o[keep], ref[keep], "f16", "decode_append_fp8 next to skipped and bad slots")
    got = [x.cpu().numpy() for x in c1]
    for g_, r_ in zip(got, (kc, vc, ks, vs)):
        assert np.array_equal(np.isnan(g_.astype(np.float64)), np.isnan(r_.astype(np.float64)))
        assert np.array_equal(np.nan_to_num(g_.astype(np.float64)), np.nan_to_num(r_.astype(np.float64)))


@pytest.mark.parametrize("cfg,kw", [(2, {}), (3, dict(median=87)), (3, dict(median=23)), (4, dict(block_size=16)),
                                    (4, dict(block_size=256))])
def test_fused_full_size(cfg, kw):
    """The benchmark's step at full size, in its launch configuration (default partitions):
    the fused append + decode against the oracle's append and decode, every output element,
    and the appended rows bit for bit."""
    dev = require_gpu()
    w = config_workload(cfg, seed=0, **kw)
    t = w.to_device(dev)
    L = int(w.lens_after_append.max())
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    note(f"fused full size cfg={cfg} {kw}")
    out = ops.decode_append(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["lens_after"], L, w.scale,
                            t["new_key"], t["new_value"], t["slot_mapping"], err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ka, va = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    ref = oracle.paged_decode(w.q, ka, va, w.block_table, w.lens_after_append, w.scale)
    assert_close(out.float().cpu().numpy(), ref, w.dtype, f"fused full size cfg {cfg} {kw}")
    blk = torch.from_numpy(w.slot_mapping // w.block_size).long().to(dev)
    off = torch.from_numpy(w.slot_mapping % w.block_size).long().to(dev)
    for pool, new in ((t["k_pool"], t["new_key"]), (t["v_pool"], t["new_value"])):
        assert torch.equal(_bits(pool[blk, :, off, :]), _bits(new)), "appended rows differ"
