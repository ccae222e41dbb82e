"""GPU: cache layouts against the oracle.

* Multi-layer caches: one allocation [blocks][2][layers][heads][bs][d] whose layer views are
  strided pools; decode, append and copy-on-write through the views, other layers untouched.
* Re-blocking (pa_reblock): every valid row moves to a layout of another block size, bit for
  bit as the oracle's re-blocking; decode over the new layout matches the oracle.
* Compaction: the block manager's plan run by pa_copy_blocks leaves every decode bitwise
  unchanged, and the pools equal the oracle's compaction.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_cache as o8
from paged_kv_cache_indexed_amd import ops
from paged_kv_cache_indexed_amd.block_manager import BlockManager
from tests.gpu_util import assert_close, note, require_gpu

pytestmark = pytest.mark.gpu

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _rounded(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(_TORCH[dtype]).float().numpy()


def _tables(rng, lens, bs, spare=5, width_extra=1):
    """Seeded placement: one permutation of the pool handed out in sequence order."""
    need = [-(-int(L) // bs) for L in lens]
    nb = sum(need) + spare
    perm = rng.permutation(nb).astype(np.int32)
    table = np.full((len(lens), max(need) + width_extra), -1, np.int32)
    cur = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[cur:cur + n]
        cur += n
    return table, nb


def _scatter(pool, table, rows, bs):
    """Write contiguous per-sequence rows [L][H][d] into their slots (indexing only)."""
    for b, r in enumerate(rows):
        t = np.arange(len(r))
        pool[table[b, t // bs], :, t % bs, :] = r


def _eq_nan(a, b):
    return np.array_equal(np.asarray(a, np.float64), np.asarray(b, np.float64), equal_nan=True)


@pytest.mark.parametrize("dtype,hkv,group,bs", [("f16", 4, 1, 16), ("bf16", 2, 8, 16), ("f32", 2, 2, 8)])
def test_multilayer_strided_cache(dtype, hkv, group, bs):
    dev = require_gpu()
    rng = np.random.default_rng([600, hkv, group])
    lens = np.array([1, 17, 64, 130, 77], np.int32)
    d, nl = 128, 3
    table, nb = _tables(rng, lens, bs)
    host = np.full((nb, 2, nl, hkv, bs, d), np.nan, np.float32)
    for layer in range(nl):
        for kv in range(2):
            rows = [_rounded(rng.standard_normal((L, hkv, d)), dtype) for L in lens]
            _scatter(host[:, kv, layer], table, rows, bs)
    q = _rounded(rng.standard_normal((len(lens), hkv * group, d)), dtype)
    cache = torch.from_numpy(host).to(_TORCH[dtype]).to(dev)
    qd = torch.from_numpy(q).to(_TORCH[dtype]).to(dev)
    td = torch.from_numpy(table).to(dev)
    ld = torch.from_numpy(lens).to(dev)
    scale = 1 / np.sqrt(d)
    for layer in range(nl):
        k, v = cache[:, 0, layer], cache[:, 1, layer]
        assert not k.is_contiguous()
        for P in (0, 2 * bs):
            note(f"multilayer {dtype} G={group} layer={layer} P={P}")
            out = ops.decode(qd, k, v, td, ld, int(lens.max()), scale, partition_size=P)
            torch.cuda.synchronize()
            ref = oracle.paged_decode(q, *oracle.layer_pools(host, layer), table, lens, scale)
            assert_close(out.float().cpu().numpy(), ref, dtype, f"multilayer layer {layer} P={P}")
    # append through layer 1's views, then copy-on-write in layer 2: nothing else may change
    key = _rounded(rng.standard_normal((len(lens), hkv, d)), dtype)
    val = _rounded(rng.standard_normal((len(lens), hkv, d)), dtype)
    slots = np.array([table[b, L // bs] * bs + L % bs for b, L in enumerate(lens)], np.int32)
    free = sorted(set(range(nb)) - set(table[table >= 0].tolist()))
    pairs = np.array([[table[2, 0], free[0]], [table[3, 1], free[1]]], np.int32)
    note(f"multilayer {dtype} append + copy through views")
    ops.reshape_and_cache(torch.from_numpy(key).to(_TORCH[dtype]).to(dev),
                          torch.from_numpy(val).to(_TORCH[dtype]).to(dev), cache[:, 0, 1], cache[:, 1, 1],
                          torch.from_numpy(slots).to(dev))
    ops.copy_blocks(cache[:, 0, 2], cache[:, 1, 2], torch.from_numpy(pairs).to(dev))
    torch.cuda.synchronize()
    want = host.copy()
    k1, v1 = oracle.reshape_and_cache(*oracle.layer_pools(host, 1), key, val, slots)
    want[:, 0, 1], want[:, 1, 1] = k1, v1
    k2, v2 = oracle.copy_blocks(*oracle.layer_pools(host, 2), pairs)
    want[:, 0, 2], want[:, 1, 2] = k2, v2
    assert _eq_nan(cache.float().cpu().numpy(), _rounded(want, dtype)), "strided append/copy wrote the wrong bytes"


def test_multilayer_fp8_cache():
    dev = require_gpu()
    rng = np.random.default_rng(610)
    lens = np.array([3, 40, 129], np.int32)
    hkv, group, d, bs, nl = 2, 4, 128, 16, 2
    table, nb = _tables(rng, lens, bs)
    codes = np.full((nb, 2, nl, hkv, bs, d), o8.E4M3_NAN_CODE, np.uint8)
    scales = np.full((nl, 2, nb, hkv, bs), np.nan, np.float32)  # dense per layer
    for layer in range(nl):
        for kv in range(2):
            rows = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
            c, s = zip(*[o8.quantize_rows(r) for r in rows])
            view = codes[:, kv, layer]
            sview = scales[layer, kv][..., None]
            _scatter(view, table, list(c), bs)
            _scatter(sview, table, [x[..., None] for x in s], bs)
    q = _rounded(rng.standard_normal((len(lens), hkv * group, d)), "bf16")
    cd = torch.from_numpy(codes).to(dev)
    sd = torch.from_numpy(scales).to(dev)
    td = torch.from_numpy(table).to(dev)
    ld = torch.from_numpy(lens).to(dev)
    qd = torch.from_numpy(q).to(torch.bfloat16).to(dev)
    for layer in range(nl):
        note(f"multilayer fp8 layer={layer}")
        out = ops.decode_fp8(qd, cd[:, 0, layer], cd[:, 1, layer], sd[layer, 0], sd[layer, 1], td, ld,
                             int(lens.max()), 0.1)
        torch.cuda.synchronize()
        ref = o8.paged_decode_fp8(q, codes[:, 0, layer], codes[:, 1, layer], scales[layer, 0], scales[layer, 1],
                                  table, lens, 0.1)
        assert_close(out.float().cpu().numpy(), ref, "bf16", f"multilayer fp8 layer {layer}")
    key = rng.standard_normal((len(lens), hkv, d)).astype(np.float32)
    slots = np.array([table[b, L // bs] * bs + L % bs for b, L in enumerate(lens)], np.int32)
    note("multilayer fp8 append through views")
    kd = torch.from_numpy(key).to(dev)
    ops.reshape_and_cache_fp8(kd, kd, cd[:, 0, 1], cd[:, 1, 1], sd[1, 0], sd[1, 1], torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    want_c, want_s = codes.copy(), scales.copy()
    r = o8.reshape_and_cache_fp8(codes[:, 0, 1], codes[:, 1, 1], scales[1, 0], scales[1, 1], key, key, slots)
    want_c[:, 0, 1], want_c[:, 1, 1], want_s[1, 0], want_s[1, 1] = r
    assert np.array_equal(cd.cpu().numpy(), want_c)
    assert _eq_nan(sd.cpu().numpy(), want_s)


@pytest.mark.parametrize("dtype,new_bs", [("f16", 8), ("f16", 32), ("bf16", 64), ("f32", 256), ("bf16", 16)])
def test_reblock_matches_oracle(dtype, new_bs):
    dev = require_gpu()
    rng = np.random.default_rng([620, new_bs])
    lens = np.array([1, 15, 16, 17, 200, 333, 0], np.int32)
    hkv, d, bs = 3, 128, 16
    table, nb = _tables(rng, lens, bs)
    pool_k = np.full((nb, hkv, bs, d), np.nan, np.float32)
    pool_v = np.full_like(pool_k, np.nan)
    _scatter(pool_k, table, [_rounded(rng.standard_normal((L, hkv, d)), dtype) for L in lens], bs)
    _scatter(pool_v, table, [_rounded(rng.standard_normal((L, hkv, d)), dtype) for L in lens], bs)
    ntab, nnb = _tables(rng, lens, new_bs, spare=2)
    live = lens > 0
    want_k = oracle.reblock(pool_k, table[live], lens[live], new_bs, ntab[live], nnb)
    want_v = oracle.reblock(pool_v, table[live], lens[live], new_bs, ntab[live], nnb)
    dt = _TORCH[dtype]
    sk, sv = torch.from_numpy(pool_k).to(dt).to(dev), torch.from_numpy(pool_v).to(dt).to(dev)
    dk = torch.full((nnb, hkv, new_bs, d), float("nan"), dtype=dt, device=dev)
    dv = torch.full_like(dk, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    note(f"reblock {dtype} 16 -> {new_bs}")
    ops.reblock(sk, sv, torch.from_numpy(table).to(dev), dk, dv, torch.from_numpy(ntab).to(dev),
                torch.from_numpy(lens).to(dev), int(lens.max()), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert _eq_nan(dk.float().cpu().numpy(), want_k) and _eq_nan(dv.float().cpu().numpy(), want_v)
    # decode over the new layout against the oracle over the old one
    q = _rounded(rng.standard_normal((int(live.sum()), hkv, d)), dtype)
    ref = oracle.paged_decode(q, pool_k, pool_v, table[live], lens[live], 0.09)
    note(f"decode after reblock {dtype} -> {new_bs}")
    out = ops.decode(torch.from_numpy(q).to(dt).to(dev), dk, dv, torch.from_numpy(ntab[live]).to(dev),
                     torch.from_numpy(lens[live]).to(dev), int(lens.max()), 0.09)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), ref, dtype, f"decode after reblock to {new_bs}")


def test_reblock_strided_source_and_fp8_scales():
    dev = require_gpu()
    rng = np.random.default_rng(630)
    lens = np.array([5, 48, 100], np.int32)
    hkv, d, bs, nl, new_bs = 2, 64, 16, 2, 32
    table, nb = _tables(rng, lens, bs)
    codes = rng.integers(0, 0x7F, (nb, 2, nl, hkv, bs, d)).astype(np.uint8)
    ks = rng.uniform(0.01, 1, (nb, hkv, bs)).astype(np.float32)
    vs = rng.uniform(0.01, 1, (nb, hkv, bs)).astype(np.float32)
    ntab, nnb = _tables(rng, lens, new_bs, spare=1)
    layer = 1
    want_kc = oracle.reblock(codes[:, 0, layer].astype(np.float32), table, lens, new_bs, ntab, nnb)
    want_vc = oracle.reblock(codes[:, 1, layer].astype(np.float32), table, lens, new_bs, ntab, nnb)
    want_ks = oracle.reblock(ks[..., None], table, lens, new_bs, ntab, nnb)[..., 0]
    want_vs = oracle.reblock(vs[..., None], table, lens, new_bs, ntab, nnb)[..., 0]
    cd = torch.from_numpy(codes).to(dev)
    dk, dv, dks, dvs = ops.empty_fp8_cache(nnb, hkv, new_bs, d, dev)
    for x in (dk, dv):
        x.fill_(0xFF)
    for x in (dks, dvs):
        x.fill_(float("nan"))
    note("reblock fp8 from a strided layer view")
    ops.reblock(cd[:, 0, layer], cd[:, 1, layer], torch.from_numpy(table).to(dev), dk, dv,
                torch.from_numpy(ntab).to(dev), torch.from_numpy(lens).to(dev), int(lens.max()),
                scales=(torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev), dks, dvs))
    torch.cuda.synchronize()
    got_kc = dk.cpu().numpy().astype(np.float32)
    written = ~np.isnan(want_kc)
    assert np.array_equal(got_kc[written], want_kc[written]) and np.all(dk.cpu().numpy()[~written] == 0xFF)
    assert np.array_equal(dv.cpu().numpy().astype(np.float32)[written], want_vc[written])
    assert _eq_nan(dks.cpu().numpy(), want_ks) and _eq_nan(dvs.cpu().numpy(), want_vs)


def test_reblock_flags_bad_ids_and_lengths():
    dev = require_gpu()
    lens = torch.tensor([20, 40], dtype=torch.int32, device=dev)
    src_t = torch.tensor([[0, 1, -1], [2, 3, 4]], dtype=torch.int32, device=dev)
    dst_t = torch.tensor([[99, 0], [1, 2]], dtype=torch.int32, device=dev)  # 99 is outside the pool
    sk = torch.zeros(6, 2, 16, 64, dtype=torch.float16, device=dev)
    dk = torch.zeros(3, 2, 32, 64, dtype=torch.float16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    note("reblock bad id")
    ops.reblock(sk, sk.clone(), src_t, dk, dk.clone(), dst_t, lens, 40, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    err.zero_()
    note("reblock bad length")
    ops.reblock(sk, sk.clone(), src_t, dk, dk.clone(), dst_t, torch.tensor([20, 70], dtype=torch.int32, device=dev),
                70, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 2


def test_compaction_keeps_every_decode():
    """Fragment a pool through the block manager, run its compaction plan on the GPU, and
    check the decode bitwise against the decode before, and the pools against the oracle."""
    dev = require_gpu()
    rng = np.random.default_rng(640)
    bs, hkv, d, nb = 16, 4, 128, 96
    bm = BlockManager(nb, bs, 32, shuffle_seed=5)
    host_k = np.full((nb, hkv, bs, d), np.nan, np.float32)
    host_v = np.full_like(host_k, np.nan)
    for sid in range(12):
        bm.add_sequence(sid)
        L = int(rng.integers(1, 90))
        slots, _ = bm.append_slots(sid, L)
        kr = _rounded(rng.standard_normal((L, hkv, d)), "f16")
        vr = _rounded(rng.standard_normal((L, hkv, d)), "f16")
        host_k, host_v = oracle.reshape_and_cache(host_k, host_v, kr, vr, slots)
    for sid in (0, 3, 4, 9):
        bm.free_sequence(sid)
    seqs = sorted(bm._seqs)
    table, lens = bm.block_table(seqs), bm.context_lens(seqs)
    q = _rounded(rng.standard_normal((len(seqs), hkv * 2, d)), "f16")
    kd = torch.from_numpy(host_k).half().to(dev)
    vd = torch.from_numpy(host_v).half().to(dev)
    qd = torch.from_numpy(q).half().to(dev)
    note("compaction: decode before")
    before = ops.decode(qd, kd, vd, torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev),
                        int(lens.max()), 0.1).clone()
    pairs = bm.compact()
    assert len(pairs) > 0 and bm.is_compact()
    new_table = bm.block_table(seqs)
    note("compaction: copy + decode after")
    ops.copy_blocks(kd, vd, torch.from_numpy(pairs).to(dev))
    after = ops.decode(qd, kd, vd, torch.from_numpy(new_table).to(dev), torch.from_numpy(lens).to(dev),
                       int(lens.max()), 0.1)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), after.view(torch.int16)), "compaction changed a decode"
    wk, wv, wt = oracle.compact_blocks(host_k, host_v, table, pairs)
    assert np.array_equal(wt, new_table)
    live = sorted(set(new_table[new_table >= 0].tolist()))
    assert _eq_nan(kd.float().cpu().numpy()[live], _rounded(wk[live], "f16"))
    assert _eq_nan(vd.float().cpu().numpy()[live], _rounded(wv[live], "f16"))
    ref = oracle.paged_decode(q, wk, wv, wt, lens, 0.1)
    assert_close(after.float().cpu().numpy(), ref, "f16", "decode after compaction")
