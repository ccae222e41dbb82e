"""GPU: multi-token paged attention (pa_multi_token_attention) against the float64 oracle.

Sequence b has n_b new query rows whose K/V are already in the cache (so context_lens[b]
includes them); query i attends causally to tokens 0 .. L_b - n_b + i.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_cache as o8
from paged_kv_cache_indexed_amd import ops
from tests.gpu_util import assert_close, note, require_gpu
from workloads import build_paged

pytestmark = pytest.mark.gpu

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def _case(name, cfg, lens, ns, bs, hkv, group, d, dtype, seed=0):
    w = build_paged(name, cfg, seed, np.asarray(lens, np.int32), bs, hkv, hkv * group, d, dtype, append=False)
    qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    rng = np.random.default_rng([cfg, seed, 9])
    q = torch.from_numpy(rng.standard_normal((int(qs[-1]), hkv * group, d)).astype(np.float32))
    q = q.to(_TORCH[dtype]).float().numpy()
    return w, qs, q


def _run(w, qs, q, dev, max_q, P=0, fp8=None, table=None):
    t = w.to_device(dev)
    dt = _TORCH[w.dtype]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kp, vp, ks, vs = (t["k_pool"], t["v_pool"], None, None) if fp8 is None else fp8
    out = ops.multi_token_attention(
        torch.from_numpy(q).to(dt).to(dev), kp, vp, t["block_table"] if table is None else table,
        t["context_lens"], torch.from_numpy(qs).to(dev), int(w.context_lens.max()), max_q, w.scale,
        k_scale=ks, v_scale=vs, partition_size=P, err_flag=err)
    torch.cuda.synchronize()
    return out, int(err.item())


@pytest.mark.parametrize("dtype,group,bs,d", [("f16", 1, 16, 128), ("bf16", 2, 32, 128), ("f16", 4, 16, 64),
                                              ("bf16", 8, 16, 128), ("f16", 16, 16, 128), ("bf16", 1, 256, 256),
                                              ("f16", 8, 64, 256), ("bf16", 8, 8, 128), ("f16", 1, 8, 64),
                                              ("f16", 16, 8, 128)])
def test_multi_token_matches_oracle(dtype, group, bs, d):
    dev = require_gpu()
    lens = [1, 16, 40, 17, 100, 300, 57]
    ns = [1, 16, 15, 17, 0, 37, 57]  # one query, a full prefill, a chunk, none, ...
    w, qs, q = _case(f"mt-{dtype}", 700 + group, lens, ns, bs, 2, group, d, dtype)
    ref = oracle.paged_attention_multi(q, w.k_pool, w.v_pool, w.block_table, w.context_lens, qs, w.scale)
    for P in [P for P in (0, 2 * bs, 128, 512) if P % bs == 0]:
        note(f"multi-token {dtype} G={group} bs={bs} d={d} P={P}")
        out, err = _run(w, qs, q, dev, max(ns), P)
        assert err == 0, f"error flag {err}"
        assert_close(out.float().cpu().numpy(), ref, dtype, f"multi-token {dtype} G={group} d={d} P={P}")


@pytest.mark.parametrize("dtype,group,d,fp8", [("bf16", 4, 128, False), ("f16", 1, 64, False), ("bf16", 8, 128, True)])
def test_multi_token_few_queries_8_token_blocks(dtype, group, d, fp8):
    """Fewer than 64 (query, head) rows per kv head over 8-token blocks: the 16-column kernel
    with a block lookup per tile row (longer chunks take the 64-row kernel, covered above)."""
    dev = require_gpu()
    lens = [1, 9, 40, 17, 100, 300]
    ns = [1, 2, 1, 0, 1, 2]
    w, qs, q = _case(f"mt-few-bs8-{dtype}", 760 + group, lens, ns, 8, 2, group, d, dtype)
    kp, vp, f8 = w.k_pool, w.v_pool, None
    if fp8:
        dead = np.isnan(w.k_pool).any(-1)
        kc, ks = o8.quantize_rows(np.nan_to_num(w.k_pool))
        vc, vs = o8.quantize_rows(np.nan_to_num(w.v_pool))
        kc[dead], vc[dead] = o8.E4M3_NAN_CODE, o8.E4M3_NAN_CODE
        ks[dead], vs[dead] = np.nan, np.nan
        kp, vp = o8.dequantize(kc, ks), o8.dequantize(vc, vs)
        f8 = tuple(torch.from_numpy(x).to(dev) for x in (kc, vc, ks, vs))
    ref = oracle.paged_attention_multi(q, kp, vp, w.block_table, w.context_lens, qs, w.scale)
    for P in (0, 8, 24, 128):
        note(f"multi-token few queries bs=8 {dtype} G={group} d={d} fp8={fp8} P={P}")
        out, err = _run(w, qs, q, dev, max(ns), P, fp8=f8)
        assert err == 0, f"error flag {err}"
        assert_close(out.float().cpu().numpy(), ref, dtype, f"few queries bs=8 G={group} d={d} P={P}")


def test_multi_token_one_query_is_the_decode_bitwise():
    """With one query per sequence the (query, head) columns are the decode's head columns,
    the partition policy is the same, and so is every bit of the output (at head_dim 64: at
    128 the decode takes its LDS path, which sums P V in 16-token steps)."""
    dev = require_gpu()
    lens = [5, 64, 333, 1000]
    w, qs, q = _case("mt-decode", 710, lens, [1, 1, 1, 1], 16, 4, 8, 64, "bf16")
    t = w.to_device(dev)
    qd = torch.from_numpy(q).to(torch.bfloat16).to(dev)
    note("multi-token n=1 vs decode")
    dec = ops.decode(qd, t["k_pool"], t["v_pool"], t["block_table"], t["context_lens"], 1000, w.scale)
    out, err = _run(w, qs, q, dev, 1)
    assert err == 0
    assert torch.equal(out.view(torch.int16), dec.view(torch.int16))


# group 1 takes the 16-column kernel; groups 4 and 8 bring 64 or more rows per kv head to
# the 64-row kernel (head_dim 64 and 128, one or two units of 8 codes per thread)
@pytest.mark.parametrize("q_dtype,group,d,bs", [("bf16", 1, 128, 16), ("f16", 8, 128, 16), ("bf16", 4, 64, 16),
                                                ("bf16", 8, 128, 32), ("f16", 4, 64, 64), ("bf16", 8, 128, 8),
                                                ("f16", 2, 64, 8)])
def test_multi_token_fp8_cache(q_dtype, group, d, bs):
    dev = require_gpu()
    lens = [20, 129, 64, 300]
    ns = [20, 7, 33, 50]
    w, qs, q = _case("mt-fp8", 720 + group, lens, ns, bs, 2, group, d, q_dtype)
    dead_k = np.isnan(w.k_pool).any(-1)
    kc, ks = o8.quantize_rows(np.nan_to_num(w.k_pool))
    vc, vs = o8.quantize_rows(np.nan_to_num(w.v_pool))
    kc[dead_k], vc[dead_k] = o8.E4M3_NAN_CODE, o8.E4M3_NAN_CODE
    ks[dead_k], vs[dead_k] = np.nan, np.nan
    ref = oracle.paged_attention_multi(q, o8.dequantize(kc, ks), o8.dequantize(vc, vs), w.block_table,
                                       w.context_lens, qs, w.scale)
    fp8 = tuple(torch.from_numpy(x).to(dev) for x in (kc, vc, ks, vs))
    for P in (0, 2 * bs):
        note(f"multi-token fp8 q={q_dtype} G={group} d={d} bs={bs} P={P}")
        out, err = _run(w, qs, q, dev, max(ns), P, fp8=fp8)
        assert err == 0
        assert_close(out.float().cpu().numpy(), ref, q_dtype, f"multi-token fp8 G={group} P={P}")


def test_multi_token_chunked_prefill_size():
    """Chunks of 128 new tokens at the end of 2048-token contexts, 32 query / 8 kv heads."""
    dev = require_gpu()
    lens = [2048] * 4
    ns = [128] * 4
    w, qs, q = _case("mt-chunk", 730, lens, ns, 16, 8, 4, 128, "bf16")
    ref = oracle.paged_attention_multi(q, w.k_pool, w.v_pool, w.block_table, w.context_lens, qs, w.scale)
    for P in (0, 256):
        note(f"chunked prefill P={P}")
        out, err = _run(w, qs, q, dev, 128, P)
        assert err == 0
        assert_close(out.float().cpu().numpy(), ref, "bf16", f"chunked prefill P={P}")


def test_multi_token_chunked_prefill_fp8():
    """The same chunks over an 8-bit cache (the 64-row kernel widening codes into its tiles)."""
    dev = require_gpu()
    lens = [2048] * 4
    ns = [128] * 4
    w, qs, q = _case("mt-chunk8", 731, lens, ns, 16, 8, 4, 128, "bf16")
    kc, ks = o8.quantize_rows(np.nan_to_num(w.k_pool))
    vc, vs = o8.quantize_rows(np.nan_to_num(w.v_pool))
    ref = oracle.paged_attention_multi(q, o8.dequantize(kc, ks), o8.dequantize(vc, vs), w.block_table,
                                       w.context_lens, qs, w.scale)
    fp8 = tuple(torch.from_numpy(x).to(dev) for x in (kc, vc, ks, vs))
    for P in (0, 256):
        note(f"chunked prefill fp8 P={P}")
        out, err = _run(w, qs, q, dev, 128, P, fp8=fp8)
        assert err == 0
        assert_close(out.float().cpu().numpy(), ref, "bf16", f"chunked prefill fp8 P={P}")


def test_multi_token_errors_poison_only_their_sequence():
    dev = require_gpu()
    lens = [30, 50, 70]
    ns = [5, 9, 3]
    w, qs, q = _case("mt-err", 740, lens, ns, 16, 2, 4, 128, "f16")
    ref = oracle.paged_attention_multi(q, w.k_pool, w.v_pool, w.block_table, w.context_lens, qs, w.scale)
    bad = torch.from_numpy(w.block_table.copy()).to(dev)
    bad[1, 2] = 1 << 30
    for P in (0, 16):
        note(f"multi-token bad block id P={P}")
        out, err = _run(w, qs, q, dev, 9, P, table=bad)
        assert err & 1
        o = out.float().cpu().numpy()
        assert np.all(np.isnan(o[qs[1]:qs[2]]))
        keep = np.r_[qs[0]:qs[1], qs[2]:qs[3]]
        assert_close(o[keep], ref[keep], "f16", f"other sequences after a bad id, P={P}")
    # more new tokens than the context holds: flagged, its rows NaN, the others exact
    w2, qs2, q2 = _case("mt-err2", 741, [4, 50], [6, 2], 16, 2, 1, 128, "f16")
    note("multi-token n > L")
    out, err = _run(w2, qs2, q2, dev, 6)
    assert err & 2
    o = out.float().cpu().numpy()
    assert np.all(np.isnan(o[:6]))
    ref2 = oracle.paged_attention_multi(q2[6:], w2.k_pool, w2.v_pool, w2.block_table[1:], w2.context_lens[1:],
                                        np.array([0, 2]), w2.scale)
    assert_close(o[6:], ref2, "f16", "the valid sequence next to n > L")


def test_multi_token_rejects_unsupported_shapes():
    dev = require_gpu()
    k = torch.zeros(4, 2, 8, 256, dtype=torch.float16, device=dev)  # 8-token blocks of 256 dims
    q = torch.zeros(3, 2, 256, dtype=torch.float16, device=dev)
    table = torch.zeros(1, 4, dtype=torch.int32, device=dev)
    lens = torch.tensor([3], dtype=torch.int32, device=dev)
    qs = torch.tensor([0, 3], dtype=torch.int32, device=dev)
    with pytest.raises(Exception):
        ops.multi_token_attention(q, k, k.clone(), table, lens, qs, 3, 3, 1.0)
    k32 = torch.zeros(4, 2, 16, 128, dtype=torch.float32, device=dev)
    with pytest.raises(Exception):
        ops.multi_token_attention(torch.zeros(3, 2, 128, dtype=torch.float32, device=dev), k32, k32.clone(), table,
                                  lens, qs, 3, 3, 1.0)
