"""GPU: beam-group decode (pa_decode_beams) against the float64 oracle and against pa_decode.

Groups of beams share the physical blocks of a common prefix and own private tail blocks;
the beam decode must give pa_decode's result for every sequence whatever the tables hold:
shared partitions are streamed once per group, divergent ones once per beam.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_cache as o8
from paged_kv_cache_indexed_amd import ops
from tests.gpu_util import assert_close, note, require_gpu
from workloads.paged import cast_like

pytestmark = pytest.mark.gpu

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def _beam_case(seed, lens, beams, hkv, group, d, bs, prefix, dtype, share=True):
    """Tables for len(lens) sequences in groups of `beams`: a group's beams list the same
    physical blocks for their first `prefix` tokens (when share), then private blocks.
    Contents are seeded N(0,1) in `dtype`; blocks no table lists hold NaN."""
    rng = np.random.default_rng([77, seed])
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    nbp = prefix // bs
    need = [-(-int(L) // bs) for L in lens]
    mbs = max(need) + 1
    groups = -(-B // beams)
    total = groups * nbp + sum(need) + 8
    perm = rng.permutation(total).astype(np.int32)
    cur = 0
    table = np.full((B, mbs), -1, np.int32)
    for g in range(groups):
        shared = perm[cur:cur + nbp]
        cur += nbp
        for b in range(g * beams, min(B, (g + 1) * beams)):
            n_sh = min(nbp, need[b]) if share else 0
            table[b, :n_sh] = shared[:n_sh]
            k = need[b] - n_sh
            table[b, n_sh:need[b]] = perm[cur:cur + k]
            cur += k
    assert cur <= total
    shape = (total, hkv, bs, d)
    k_pool = np.full(shape, np.nan, np.float32)
    v_pool = np.full(shape, np.nan, np.float32)
    used = np.unique(table[table >= 0])
    k_pool[used] = cast_like(rng.standard_normal((len(used), hkv, bs, d)).astype(np.float32), dtype)
    v_pool[used] = cast_like(rng.standard_normal((len(used), hkv, bs, d)).astype(np.float32), dtype)
    q = cast_like(rng.standard_normal((B, hkv * group, d)).astype(np.float32), dtype)
    return q, k_pool, v_pool, table, lens


def _device(dev, dtype, q, k_pool, v_pool, table, lens):
    dt = _TORCH[dtype]
    return (torch.from_numpy(q).to(dt).to(dev), torch.from_numpy(k_pool).to(dt).to(dev),
            torch.from_numpy(v_pool).to(dt).to(dev), torch.from_numpy(table).to(dev),
            torch.from_numpy(lens).to(dev))


# lengths: a full group past the shared prefix, one with beams shorter than the prefix, and
# a last group of two beams
_LENS = [300, 290, 331, 257, 100, 200, 256, 270, 45, 333]


@pytest.mark.parametrize("dtype,group,beams,d,bs", [("bf16", 1, 4, 128, 32), ("f16", 2, 4, 64, 16),
                                                     ("bf16", 4, 4, 128, 16), ("bf16", 8, 2, 128, 16),
                                                     ("f16", 1, 16, 128, 16), ("bf16", 4, 4, 128, 8),
                                                     ("f16", 2, 4, 64, 8)])
def test_beams_match_oracle(dtype, group, beams, d, bs):
    dev = require_gpu()
    lens = _LENS if beams <= 4 else _LENS + [250, 256, 260, 261, 262, 263]
    q, kp, vp, table, L = _beam_case(1, lens, beams, 2, group, d, bs, 256, dtype)
    ref = oracle.paged_decode(q, kp, vp, table, L, 1.0 / np.sqrt(d))
    tq, tk, tv, tt, tl = _device(dev, dtype, q, kp, vp, table, L)
    for P in (0, 64, 128, 512):
        note(f"beams {dtype} G={group} W={beams} d={d} bs={bs} P={P}")
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        out = ops.decode_beams(tq, tk, tv, tt, tl, int(L.max()), 1.0 / np.sqrt(d), beams, partition_size=P,
                               err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert_close(out.float().cpu().numpy(), ref, dtype, f"beams G={group} W={beams} P={P}")


@pytest.mark.parametrize("group,bs", [(4, 16), (8, 16), (8, 8)])
def test_beams_bitwise_equal_to_grouped_decode(group, bs):
    """With 4 or 8 query heads per kv head at head_dim 64 pa_decode runs the same matrix-core
    arithmetic per column, so for an explicit partition size the outputs agree bit for bit,
    shared or not (with 8-token blocks too, where the two load the rows in different ways).
    (At head_dim 128 pa_decode takes its LDS path, which sums P V in 16-token steps; the beam
    kernel is checked against the oracle there.)"""
    dev = require_gpu()
    for share in (True, False):
        q, kp, vp, table, L = _beam_case(2, _LENS, 2, 2, group, 64, bs, 256, "bf16", share=share)
        tq, tk, tv, tt, tl = _device(dev, "bf16", q, kp, vp, table, L)
        for P in (64, 256):
            note(f"beams vs decode G={group} share={share} P={P}")
            a = ops.decode(tq, tk, tv, tt, tl, int(L.max()), 0.125, partition_size=P)
            b = ops.decode_beams(tq, tk, tv, tt, tl, int(L.max()), 0.125, 2, partition_size=P)
            torch.cuda.synchronize()
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_beams_degenerate_groups():
    """beam_width 1 (every sequence its own group) and the largest partition the staged table
    slices allow (beam_width x P / block_size = 2048 ids)."""
    dev = require_gpu()
    q, kp, vp, table, L = _beam_case(7, _LENS, 4, 2, 1, 64, 16, 256, "f16")
    ref = oracle.paged_decode(q, kp, vp, table, L, 0.125)
    tq, tk, tv, tt, tl = _device(dev, "f16", q, kp, vp, table, L)
    for W, P in ((1, 0), (1, 16 * 2048), (4, 16 * 512), (4, 16)):
        note(f"beams W={W} P={P}")
        out = ops.decode_beams(tq, tk, tv, tt, tl, int(L.max()), 0.125, W, partition_size=P)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy(), ref, "f16", f"beams W={W} P={P}")
    with pytest.raises(Exception):  # 4 beams x 513 ids of a partition: over the staged slices
        ops.decode_beams(tq, tk, tv, tt, tl, int(L.max()), 0.125, 4, partition_size=16 * 513)
    # a loose max_context_len: most partitions of the launch lie past every beam of a group
    wide = torch.full((tt.shape[0], 4 * tt.shape[1]), -1, dtype=torch.int32, device=dev)
    wide[:, :tt.shape[1]] = tt
    note("beams loose max_context_len")
    out = ops.decode_beams(tq, tk, tv, wide, tl, 4 * int(L.max()), 0.125, 4, partition_size=64)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), ref, "f16", "beams loose max_context_len")


def test_beams_private_tables():
    """No block is shared: every partition takes the per-beam passes."""
    dev = require_gpu()
    q, kp, vp, table, L = _beam_case(3, _LENS, 4, 2, 1, 128, 32, 256, "bf16", share=False)
    ref = oracle.paged_decode(q, kp, vp, table, L, 0.1)
    tq, tk, tv, tt, tl = _device(dev, "bf16", q, kp, vp, table, L)
    for P in (0, 96):
        note(f"beams private tables P={P}")
        out = ops.decode_beams(tq, tk, tv, tt, tl, int(L.max()), 0.1, 4, partition_size=P)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy(), ref, "bf16", f"beams private tables P={P}")


@pytest.mark.parametrize("q_dtype,bs", [("bf16", 32), ("f16", 32), ("bf16", 8)])
def test_beams_fp8_cache(q_dtype, bs):
    dev = require_gpu()
    q, kp, vp, table, L = _beam_case(4, _LENS, 4, 2, 1, 128, bs, 256, q_dtype)
    dead = np.isnan(kp).any(-1)
    kc, ks = o8.quantize_rows(np.nan_to_num(kp))
    vc, vs = o8.quantize_rows(np.nan_to_num(vp))
    kc[dead], vc[dead] = o8.E4M3_NAN_CODE, o8.E4M3_NAN_CODE
    ks[dead], vs[dead] = np.nan, np.nan
    ref = oracle.paged_decode(q, o8.dequantize(kc, ks), o8.dequantize(vc, vs), table, L, 0.09)
    t8 = [torch.from_numpy(x).to(dev) for x in (kc, vc, ks, vs)]
    tq = torch.from_numpy(q).to(_TORCH[q_dtype]).to(dev)
    tt, tl = torch.from_numpy(table).to(dev), torch.from_numpy(L).to(dev)
    for P in (0, 128):
        note(f"beams fp8 q={q_dtype} bs={bs} P={P}")
        out = ops.decode_beams(tq, t8[0], t8[1], tt, tl, int(L.max()), 0.09, 4, k_scale=t8[2], v_scale=t8[3],
                               partition_size=P)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy(), ref, q_dtype, f"beams fp8 P={P}")


def test_beams_errors_poison_only_their_sequence():
    dev = require_gpu()
    q, kp, vp, table, L = _beam_case(5, _LENS, 4, 2, 1, 128, 32, 256, "bf16")
    ref = oracle.paged_decode(q, kp, vp, table, L, 0.1)
    tq, tk, tv, tt, tl = _device(dev, "bf16", q, kp, vp, table, L)
    cases = [("bad id in a private tail", 1, 9, 1), ("bad id inside the shared prefix", 2, 3, 1),
             ("bad length", 6, None, 2)]
    for what, b, j, flag in cases:
        bad_t, bad_l = tt.clone(), tl.clone()
        if j is None:
            bad_l[b] = 1 << 20
        else:
            bad_t[b, j] = 1 << 30
        for P in (0, 64):
            note(f"beams {what} (sequence {b}) P={P}")
            err = torch.zeros(1, dtype=torch.int32, device=dev)
            out = ops.decode_beams(tq, tk, tv, bad_t, bad_l, int(L.max()), 0.1, 4, partition_size=P,
                                   err_flag=err)
            torch.cuda.synchronize()
            assert int(err.item()) & flag, what
            o = out.float().cpu().numpy()
            assert np.all(np.isnan(o[b])), what
            keep = [i for i in range(len(L)) if i != b]
            assert_close(o[keep], ref[keep], "bf16", f"other sequences after {what}, P={P}")


def test_beams_rejects_unsupported_shapes():
    dev = require_gpu()
    q, kp, vp, table, L = _beam_case(6, [40, 50], 2, 2, 1, 256, 16, 16, "bf16")
    tq, tk, tv, tt, tl = _device(dev, "bf16", q, kp, vp, table, L)
    with pytest.raises(Exception):  # head_dim 256
        ops.decode_beams(tq, tk, tv, tt, tl, 50, 0.1, 2)
    q, kp, vp, table, L = _beam_case(6, [40, 50], 2, 2, 8, 128, 16, 16, "bf16")
    tq, tk, tv, tt, tl = _device(dev, "bf16", q, kp, vp, table, L)
    with pytest.raises(Exception):  # 8 heads per kv head x 4 beams: more than 16 columns
        ops.decode_beams(tq, tk, tv, tt, tl, 50, 0.1, 4)
