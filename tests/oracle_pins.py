"""Pins for the CPU oracle: facts fixed by the pages and by mathematics, not by the oracle.

Every pin takes the oracle module ``o`` as its argument so that the mutation test can run
the very same pins against planted mistakes (tests/test_oracle_mutations.py). A pin raises
AssertionError when the implementation disagrees with the fact it checks.

Sources of truth used here:
  * brute force on tiny inputs: contiguous K/V scattered into a pool by a per-element loop,
    and attention evaluated with scalar Python loops (``math.exp``);
  * closed forms: identical keys, a dominant key, a single key, a zero scale;
  * invariants: uniform score shift, linearity in V, GQA as replicated MHA, joint token
    permutation, physical relabelling of blocks, block-size independence, NaN padding;
  * a library routine: torch's CPU scaled_dot_product_attention in float64;
  * the pages' printed numbers (tests/golden/*.json, each with its citation).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(*key):
    return np.random.default_rng(list(key))


def _scatter_loop(contents, bs, ids, num_blocks, dtype=np.float32):
    """Brute-force paging: token t of ``contents`` [L][H][d] goes to (ids[t // bs], h, t % bs)."""
    L, H, d = contents.shape
    pool = np.full((num_blocks, H, bs, d), np.nan, dtype)
    for t in range(L):
        for h in range(H):
            for e in range(d):
                pool[ids[t // bs], h, t % bs, e] = contents[t, h, e]
    return pool


def _make_case(seed, lens, Hq, Hkv, d, bs, spare=3, table_width=None, std=1.0):
    """Tiny paged case: contiguous contents, shuffled ids, NaN-poisoned unused slots."""
    rng = _rng(seed, bs, d)
    lens = [int(x) for x in lens]
    B = len(lens)
    kc = [(rng.standard_normal((L, Hkv, d)) * std).astype(np.float32) for L in lens]
    vc = [(rng.standard_normal((L, Hkv, d)) * std).astype(np.float32) for L in lens]
    q = (rng.standard_normal((B, Hq, d)) * std).astype(np.float32)
    nbs = [-(-L // bs) for L in lens]
    num_blocks = sum(nbs) + spare
    perm = rng.permutation(num_blocks)
    width = table_width or max(nbs) + 1
    table = np.full((B, width), -1, np.int32)
    cur = 0
    k_pool = np.full((num_blocks, Hkv, bs, d), np.nan, np.float32)
    v_pool = np.full_like(k_pool, np.nan)
    for b in range(B):
        ids = perm[cur:cur + nbs[b]]
        cur += nbs[b]
        table[b, :nbs[b]] = ids
        for t in range(lens[b]):
            k_pool[ids[t // bs], :, t % bs, :] = kc[b][t]
            v_pool[ids[t // bs], :, t % bs, :] = vc[b][t]
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, table=table, lens=np.array(lens, np.int32),
                kc=kc, vc=vc, Hq=Hq, Hkv=Hkv, d=d, bs=bs)


def _brute_decode(q, kc, vc, lens, scale, Hq, Hkv):
    """Attention from contiguous per-sequence K/V with scalar Python arithmetic."""
    B = len(lens)
    d = q.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = []
            for t in range(int(lens[b])):
                acc = 0.0
                for e in range(d):
                    acc += float(q[b, h, e]) * float(kc[b][t, g, e])
                s.append(scale * acc)
            m = max(s)
            w = [math.exp(x - m) for x in s]
            den = sum(w)
            for e in range(d):
                out[b, h, e] = sum(w[t] * float(vc[b][t, g, e]) for t in range(len(w))) / den
    return out


def _decode(o, c, scale, **over):
    a = dict(q=c["q"], k_pool=c["k_pool"], v_pool=c["v_pool"], table=c["table"], lens=c["lens"])
    a.update(over)
    return o.paged_decode(a["q"], a["k_pool"], a["v_pool"], a["table"], a["lens"], scale)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------- pins

def pin_gather_roundtrip(o):
    """Gathering through a random table returns the contiguous rows bit for bit."""
    for i, (bs, L, H, d) in enumerate([(4, 1, 2, 3), (4, 4, 1, 2), (4, 11, 2, 3), (8, 17, 3, 2),
                                       (16, 16, 1, 4), (2, 9, 2, 2), (1, 5, 2, 2)]):
        rng = _rng(100 + i)
        contents = rng.standard_normal((L, H, d)).astype(np.float32)
        nb = -(-L // bs)
        ids = rng.permutation(nb + 5)[:nb]
        pool = _scatter_loop(contents, bs, ids, nb + 5)
        row = np.full(nb + 2, -1, np.int32)
        row[:nb] = ids
        for h in range(H):
            got = o.gather_sequence(pool, row, L, h)
            assert got.dtype == np.float64, "gather must upcast to float64"
            assert got.shape == (L, d), f"gather shape {got.shape} != {(L, d)}"
            assert np.array_equal(got, contents[:, h].astype(np.float64)), \
                f"gather mismatch bs={bs} L={L} head={h}"


def pin_worked_example(o):
    """[BlockManager essay] section 2: lengths [32,128,64,96] in 16-token blocks."""
    g = _golden("worked_example_blockmanager_s2.json")
    bs = g["block_size"]
    counts = [o.blocks_needed(L, bs) for L in g["context_lens"]]
    assert sum(g["context_lens"]) == g["total_tokens"]
    assert counts[g["request_index_128_tokens"]] == g["request_128_num_blocks"]
    assert counts == [2, 8, 4, 6] and sum(counts) == 20, f"block counts {counts}"
    ids = np.array(g["request_128_block_ids"], np.int32)
    rng = _rng(7)
    contents = rng.standard_normal((128, 2, 4)).astype(np.float32)
    pool = _scatter_loop(contents, bs, ids, 100)  # every other block stays NaN
    for h in range(2):
        got = o.gather_sequence(pool, ids, 128, h)
        assert np.array_equal(got, contents[:, h].astype(np.float64)), "worked-example gather"


def pin_memory_formula(o):
    """Closed-form sizes printed by the pages (tests/golden/kv_sizes.json)."""
    g = _golden("kv_sizes.json")
    t = g["per_token"]
    assert o.kv_cache_bytes(t["num_kv_heads"], t["head_dim"], t["dtype_bytes"], [1]) == t["bytes"]
    b = g["per_block"]
    assert o.kv_cache_bytes(b["num_kv_heads"], b["head_dim"], b["dtype_bytes"], [b["block_size"]],
                            num_layers=b["num_layers"]) == b["bytes"]
    w = g["worked_example_fp32"]
    assert o.kv_cache_bytes(w["num_kv_heads"], w["head_dim"], w["dtype_bytes"],
                            w["context_lens"]) == w["bytes"]
    p = g["preallocation_7b"]
    assert o.kv_cache_bytes(p["num_kv_heads"], p["head_dim"], p["dtype_bytes"],
                            [p["tokens_per_seq"]] * p["batch"], num_layers=p["num_layers"]) == p["bytes"]
    # sum over sequences, and whole blocks for the allocated figure
    lens = [33, 16, 1]
    assert o.kv_cache_bytes(8, 64, 4, lens) == sum(o.kv_cache_bytes(8, 64, 4, [L]) for L in lens)
    assert o.allocated_kv_bytes(8, 64, 4, lens, 16) == 2 * 8 * 64 * 4 * 16 * (3 + 1 + 1)


def pin_bruteforce(o):
    """Paged decode equals scalar-loop attention over the contiguous K/V (tiny inputs)."""
    for seed, lens, Hq, Hkv, d, bs in [(1, [1, 7, 12], 4, 2, 5, 4), (2, [5, 2], 3, 3, 4, 2),
                                       (3, [9, 16], 4, 1, 3, 8), (4, [3], 2, 2, 2, 1)]:
        c = _make_case(seed, lens, Hq, Hkv, d, bs)
        scale = 1.0 / math.sqrt(d)
        got = _decode(o, c, scale)
        ref = _brute_decode(c["q"], c["kc"], c["vc"], c["lens"], scale, Hq, Hkv)
        _close(got, ref, 1e-12, f"brute force seed={seed}")
        pairs = [(b, h) for b in range(len(lens)) for h in range(Hq)][::3]
        sub = o.paged_decode_heads(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], scale, pairs)
        _close(sub, np.array([ref[b, h] for b, h in pairs]), 1e-12, f"listed heads seed={seed}")


def pin_closed_forms(o):
    d, L, bs = 6, 13, 4
    c = _make_case(11, [L], 2, 2, d, bs)
    rng = _rng(12)
    # (a) identical keys: equal weights, output = mean of V
    kc = np.repeat(rng.standard_normal((1, 2, d)).astype(np.float32), L, axis=0)
    cc = _make_case(11, [L], 2, 2, d, bs)
    ids = cc["table"][0, :4]
    kp = _scatter_loop(kc, bs, ids, cc["k_pool"].shape[0])
    got = _decode(o, cc, 0.7, k_pool=kp)
    for h in range(2):
        _close(got[0, h], cc["vc"][0][:, h].astype(np.float64).mean(0), 1e-13, "identical keys")
    # (b) one dominant key: score gap >= 40 returns that key's value
    q = c["q"][0, 0].astype(np.float64)
    j = 5
    kc = (rng.standard_normal((L, 2, d)) * 0.01).astype(np.float32)
    kc[j, 0] = (q * (60.0 / float(q @ q))).astype(np.float32)
    kp = _scatter_loop(kc, bs, c["table"][0, :4], c["k_pool"].shape[0])
    s = kc[:, 0].astype(np.float64) @ q
    assert s[j] - np.max(np.delete(s, j)) >= 40.0
    got = _decode(o, c, 1.0, k_pool=kp)
    _close(got[0, 0], c["vc"][0][j, 0], 1e-12, "dominant key")
    # (c) a single key returns its value exactly
    c1 = _make_case(13, [1], 2, 1, d, bs)
    got = _decode(o, c1, 0.3)
    for h in range(2):
        assert np.array_equal(got[0, h], c1["vc"][0][0, 0].astype(np.float64)), "L = 1"
    # (d) zero scale: uniform weights
    got = _decode(o, c, 0.0)
    for h in range(2):
        _close(got[0, h], c["vc"][0][:, h].astype(np.float64).mean(0), 1e-13, "zero scale")


def pin_invariants(o):
    lens, Hq, Hkv, d, bs = [6, 11, 1], 4, 2, 5, 4
    c = _make_case(21, lens, Hq, Hkv, d, bs)
    scale = 0.45
    base = _decode(o, c, scale)
    nb = c["k_pool"].shape[0]
    rng = _rng(22)

    def rescatter(kc_list, bs_=bs, table=None, num_blocks=nb, dtype=np.float32):
        table = c["table"] if table is None else table
        pool = np.full((num_blocks, Hkv, bs_, d), np.nan, dtype)
        for b, L in enumerate(lens):
            part = _scatter_loop(kc_list[b], bs_, table[b][:-(-L // bs_)], num_blocks, dtype)
            m = ~np.isnan(part)
            pool[m] = part[m]
        return pool

    # (a) adding one vector to every key of a head shifts all its scores equally, so the
    # output does not move (float64 pools keep the shift exact up to fp64 rounding)
    u = rng.standard_normal((Hkv, d))
    shifted = [k.astype(np.float64) + u for k in c["kc"]]
    got = _decode(o, c, scale, k_pool=rescatter(shifted, dtype=np.float64))
    _close(got, base, 1e-12, "uniform key shift")
    # (b) linear in V
    v2 = [rng.standard_normal(v.shape) for v in c["vc"]]
    comb = [2.0 * a.astype(np.float64) - 0.5 * b2 for a, b2 in zip(c["vc"], v2)]
    out2 = _decode(o, c, scale, v_pool=rescatter(v2, dtype=np.float64))
    outc = _decode(o, c, scale, v_pool=rescatter(comb, dtype=np.float64))
    _close(outc, 2.0 * base - 0.5 * out2, 1e-12, "linearity in V")
    # (c) GQA equals MHA with each kv head replicated for its query heads
    rep_k = [np.repeat(k, Hq // Hkv, axis=1) for k in c["kc"]]
    rep_v = [np.repeat(v, Hq // Hkv, axis=1) for v in c["vc"]]
    kp = np.full((nb, Hq, bs, d), np.nan, np.float32)
    vp = np.full_like(kp, np.nan)
    for b, L in enumerate(lens):
        ids = c["table"][b][:-(-L // bs)]
        for t in range(L):
            kp[ids[t // bs], :, t % bs] = rep_k[b][t]
            vp[ids[t // bs], :, t % bs] = rep_v[b][t]
    mha = _decode(o, c, scale, k_pool=kp, v_pool=vp)
    assert np.array_equal(mha, base), "GQA != replicated MHA"
    # (d) joint permutation of a sequence's tokens
    perm = [rng.permutation(L) for L in lens]
    pk = [k[p] for k, p in zip(c["kc"], perm)]
    pv = [v[p] for v, p in zip(c["vc"], perm)]
    got = _decode(o, c, scale, k_pool=rescatter(pk), v_pool=rescatter(pv))
    _close(got, base, 1e-12, "token permutation")
    # (e) relabelling physical blocks leaves the result bit-identical
    pi = rng.permutation(nb)
    kp2 = np.empty_like(c["k_pool"])
    vp2 = np.empty_like(c["v_pool"])
    kp2[pi] = c["k_pool"]
    vp2[pi] = c["v_pool"]
    t2 = np.where(c["table"] >= 0, pi[np.maximum(c["table"], 0)], -1).astype(np.int32)
    assert np.array_equal(_decode(o, c, scale, k_pool=kp2, v_pool=vp2, table=t2), base), "relabel"
    # (f) the same contents under other block sizes give bit-identical results
    for bs2 in (1, 2, 8, 16):
        nb2 = sum(-(-L // bs2) for L in lens) + 2
        ids_all = rng.permutation(nb2)
        table2 = np.full((len(lens), max(-(-L // bs2) for L in lens) + 1), -1, np.int32)
        cur = 0
        kp3 = np.full((nb2, Hkv, bs2, d), np.nan, np.float32)
        vp3 = np.full_like(kp3, np.nan)
        for b, L in enumerate(lens):
            n = -(-L // bs2)
            table2[b, :n] = ids_all[cur:cur + n]
            cur += n
            for t in range(L):
                kp3[table2[b, t // bs2], :, t % bs2] = c["kc"][b][t]
                vp3[table2[b, t // bs2], :, t % bs2] = c["vc"][b][t]
        got = _decode(o, c, scale, k_pool=kp3, v_pool=vp3, table=table2)
        assert np.array_equal(got, base), f"block size {bs2} changes the result"
    # (g) garbage ids past the valid blocks and NaN padding are never read
    t3 = c["table"].copy()
    t3[:, -1] = 10 ** 6
    t3[2, 1:] = -5
    got = _decode(o, c, scale, table=t3)
    assert np.array_equal(got, base) and np.all(np.isfinite(got)), "padding / unused ids were read"


def pin_sdpa(o):
    """torch CPU scaled_dot_product_attention in float64 on the contiguous K/V."""
    import torch

    lens, Hq, Hkv, d, bs = [9, 4, 17], 6, 3, 8, 4
    c = _make_case(31, lens, Hq, Hkv, d, bs)
    scale = 0.31
    got = _decode(o, c, scale)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        q = torch.from_numpy(c["q"][b].astype(np.float64)).view(1, Hq, 1, d)
        k = torch.from_numpy(np.repeat(c["kc"][b], G, axis=1).astype(np.float64)).permute(1, 0, 2)
        v = torch.from_numpy(np.repeat(c["vc"][b], G, axis=1).astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k.unsqueeze(0).contiguous(), v.unsqueeze(0).contiguous(), scale=scale)
        _close(got[b], ref.view(Hq, d).numpy(), 1e-12, f"sdpa seq {b}")


def pin_reshape_and_cache(o):
    rng = _rng(41)
    NB, H, bs, d = 7, 2, 4, 3
    kp = rng.standard_normal((NB, H, bs, d)).astype(np.float32)
    vp = rng.standard_normal((NB, H, bs, d)).astype(np.float32)
    key = rng.standard_normal((5, H, d)).astype(np.float32)
    val = rng.standard_normal((5, H, d)).astype(np.float32)
    slots = np.array([3, -1, 27, 8, -7], np.int32)
    ek, ev = kp.copy(), vp.copy()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        for h in range(H):
            for e in range(d):
                ek[s // bs, h, s % bs, e] = key[i, h, e]
                ev[s // bs, h, s % bs, e] = val[i, h, e]
    k2, v2 = o.reshape_and_cache(kp, vp, key, val, slots)
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev), "reshape_and_cache scatter"
    assert not np.array_equal(k2, kp), "pools must be updated"
    k3, v3 = o.reshape_and_cache(kp, vp, key, val, np.full(5, -1, np.int32))
    assert np.array_equal(k3, kp) and np.array_equal(v3, vp), "negative slots must be skipped"
    try:
        o.reshape_and_cache(kp, vp, key[:1], val[:1], np.array([NB * bs], np.int32))
    except ValueError:
        pass
    else:
        raise AssertionError("slot beyond the pool must raise")


def pin_copy_blocks(o):
    rng = _rng(51)
    NB = 8
    kp = rng.standard_normal((NB, 2, 4, 3)).astype(np.float32)
    vp = rng.standard_normal((NB, 2, 4, 3)).astype(np.float32)
    pairs = np.array([[1, 4], [2, 6]], np.int32)
    k2, v2 = o.copy_blocks(kp, vp, pairs)
    ek, ev = kp.copy(), vp.copy()
    ek[4], ev[4], ek[6], ev[6] = kp[1], vp[1], kp[2], vp[2]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev), "copy_blocks"
    for bad in ([1, 1], [-1, 2], [0, NB]):
        try:
            o.copy_blocks(kp, vp, np.array([bad], np.int32))
        except ValueError:
            continue
        raise AssertionError(f"bad pair {bad} must raise")


def pin_errors(o):
    c = _make_case(61, [6, 9], 2, 2, 3, 4)
    t = c["table"].copy()
    t[1, 1] = c["k_pool"].shape[0]  # an id outside the pool inside the valid range
    for over, what in [(dict(table=t), "bad block id"),
                       (dict(lens=np.array([6, 0], np.int32)), "zero length"),
                       (dict(lens=np.array([6, 4 * c["table"].shape[1] + 1], np.int32)), "over capacity")]:
        try:
            _decode(o, c, 0.5, **over)
        except ValueError:
            continue
        raise AssertionError(f"{what} must raise")


def pin_sliding_window(o):
    """Window decode: brute force over the last W tokens; W >= L is the full decode bit for
    bit; W = 1 returns the last value; blocks wholly before the window may be -1."""
    lens, Hq, Hkv, d, bs = [1, 7, 13, 20], 4, 2, 5, 4
    c = _make_case(71, lens, Hq, Hkv, d, bs)
    scale = 0.4
    full = _decode(o, c, scale)
    for W in (1, 3, 4, 5, 12, 19, 20, 50):
        got = o.paged_decode_window(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], scale, W)
        kc = [k[max(0, L - W):] for k, L in zip(c["kc"], lens)]
        vc = [v[max(0, L - W):] for v, L in zip(c["vc"], lens)]
        ref = _brute_decode(c["q"], kc, vc, [min(L, W) for L in lens], scale, Hq, Hkv)
        _close(got, ref, 1e-12, f"window {W}")
        if W >= max(lens):
            assert np.array_equal(got, full), "window >= L must equal the full decode"
        # blocks that lie wholly before the window are released: -1 there is never read
        t = c["table"].copy()
        for b, L in enumerate(lens):
            t[b, :max(0, L - W) // bs] = -1
        got2 = o.paged_decode_window(c["q"], c["k_pool"], c["v_pool"], t, c["lens"], scale, W)
        assert np.array_equal(got2, got), "released blocks before the window were read"
    last = o.paged_decode_window(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], scale, 1)
    for b, L in enumerate(lens):
        for h in range(Hq):
            assert np.array_equal(last[b, h], c["vc"][b][L - 1, h // (Hq // Hkv)].astype(np.float64))


def pin_multilayer_pools(o):
    """One allocation [blocks][2][layers][heads][bs][d] (K/V in dim 1): each layer's pools,
    taken as views, decode to the brute force over that layer's contiguous contents."""
    lens, Hq, Hkv, d, bs, nl = [3, 9, 14], 4, 2, 4, 4, 3
    rng = _rng(81)
    nbs = [-(-L // bs) for L in lens]
    nb = sum(nbs) + 2
    perm = rng.permutation(nb)
    table = np.full((len(lens), max(nbs)), -1, np.int32)
    cur = 0
    for b, n in enumerate(nbs):
        table[b, :n] = perm[cur:cur + n]
        cur += n
    cache = np.full((nb, 2, nl, Hkv, bs, d), np.nan, np.float64)
    contents = {}
    for layer in range(nl):
        for kv in range(2):
            for b, L in enumerate(lens):
                x = rng.standard_normal((L, Hkv, d))
                contents[(layer, kv, b)] = x
                for t in range(L):
                    for h in range(Hkv):
                        for e in range(d):
                            cache[table[b, t // bs], kv, layer, h, t % bs, e] = x[t, h, e]
    q = rng.standard_normal((len(lens), Hq, d))
    for layer in range(nl):
        k, v = o.layer_pools(cache, layer)
        assert k.shape == (nb, Hkv, bs, d) and np.shares_memory(k, cache)
        assert k.strides[0] == 2 * nl * Hkv * bs * d * 8, "blocks are 2 x layers slabs apart"
        got = o.paged_decode(q, k, v, table, np.array(lens), 0.5)
        ref = _brute_decode(q, [contents[(layer, 0, b)] for b in range(len(lens))],
                            [contents[(layer, 1, b)] for b in range(len(lens))], lens, 0.5, Hq, Hkv)
        _close(got, ref, 1e-12, f"layer {layer}")


def pin_reblock(o):
    """Re-blocking moves every valid row, in order, into the new tables' blocks of the new
    size: each sequence gathers back to its contiguous contents bit for bit, nothing else is
    written, and the decode is bitwise unchanged."""
    lens, Hq, Hkv, d, bs = [1, 4, 7, 13], 2, 2, 3, 4
    c = _make_case(82, lens, Hq, Hkv, d, bs)
    base = o.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], 0.7)
    for nbs in (1, 2, 8, 16):
        need = [-(-L // nbs) for L in lens]
        nnb = sum(need) + 3
        perm = _rng(83, nbs).permutation(nnb)
        ntab = np.full((len(lens), max(need) + 1), -1, np.int32)
        cur = 0
        for b, n in enumerate(need):
            ntab[b, :n] = perm[cur:cur + n]
            cur += n
        nk = o.reblock(c["k_pool"], c["table"], c["lens"], nbs, ntab, nnb)
        nv = o.reblock(c["v_pool"], c["table"], c["lens"], nbs, ntab, nnb)
        assert nk.shape == (nnb, Hkv, nbs, d)
        for b, L in enumerate(lens):
            for h in range(Hkv):
                assert np.array_equal(o.gather_sequence(nk, ntab[b], L, h), c["kc"][b][:, h].astype(np.float64))
                assert np.array_equal(o.gather_sequence(nv, ntab[b], L, h), c["vc"][b][:, h].astype(np.float64))
        assert np.count_nonzero(~np.isnan(nk[..., 0])) == sum(lens) * Hkv, "only valid rows are written"
        got = o.paged_decode(c["q"], nk, nv, ntab, c["lens"], 0.7)
        assert np.array_equal(got, base), f"decode changed by re-blocking to {nbs}"
    bad = np.full((len(lens), 1), 0, np.int32)
    try:
        o.reblock(c["k_pool"], c["table"], c["lens"], 4, bad, 10)
    except o.OracleInputError:
        pass
    else:
        raise AssertionError("a new table too narrow for the lengths must raise")


def pin_compact_blocks(o):
    """Compaction: live blocks move to the lowest ids, tables are rewritten, and the decode
    and every gathered sequence are bitwise unchanged."""
    lens, Hq, Hkv, d, bs = [5, 9, 2, 12], 4, 2, 4, 4
    c = _make_case(84, lens, Hq, Hkv, d, bs, spare=7)
    live = sorted({int(x) for x in c["table"].ravel() if x >= 0})
    n_live = len(live)
    free_low = [i for i in range(n_live) if i not in live]
    high = [i for i in live if i >= n_live]
    pairs = np.array(list(zip(high, free_low)), np.int32).reshape(-1, 2)
    assert len(pairs) > 0
    base = o.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], 0.4)
    k2, v2, t2 = o.compact_blocks(c["k_pool"], c["v_pool"], c["table"], pairs)
    assert {int(x) for x in t2.ravel() if x >= 0} == set(range(n_live)), "live blocks must end up in [0, n_live)"
    assert np.array_equal(t2 < 0, c["table"] < 0)
    got = o.paged_decode(c["q"], k2, v2, t2, c["lens"], 0.4)
    assert np.array_equal(got, base), "compaction changed the decode"
    for b, L in enumerate(lens):
        for h in range(Hkv):
            assert np.array_equal(o.gather_sequence(k2, t2[b], L, h), c["kc"][b][:, h].astype(np.float64))


def pin_multi_token(o):
    """Several queries per sequence: one query equals the decode; a whole sequence of queries
    equals torch's causal scaled_dot_product_attention (float64, CPU); brute force on tiny
    cases; and a query's output does not depend on tokens after its position."""
    import torch

    lens, Hq, Hkv, d, bs = [1, 6, 11, 16], 4, 2, 8, 4
    c = _make_case(85, lens, Hq, Hkv, d, bs)
    scale = 0.45
    rng = _rng(86)
    # n = 1: the single-query decode, bit for bit
    qs1 = np.arange(len(lens) + 1)
    got = o.paged_attention_multi(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], qs1, scale)
    assert np.array_equal(got, o.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["table"], c["lens"], scale))
    # mixed query counts against brute force over the causal prefix
    ns = [1, 3, 0, 16]
    qs = np.concatenate([[0], np.cumsum(ns)])
    q = rng.standard_normal((int(qs[-1]), Hq, d))
    got = o.paged_attention_multi(q, c["k_pool"], c["v_pool"], c["table"], c["lens"], qs, scale)
    for b, (L, n) in enumerate(zip(lens, ns)):
        for i in range(n):
            p = L - n + i
            ref = _brute_decode(q[qs[b] + i][None], [c["kc"][b][:p + 1]], [c["vc"][b][:p + 1]], [p + 1], scale,
                                Hq, Hkv)[0]
            _close(got[qs[b] + i], ref, 1e-12, f"seq {b} query {i}")
    # n = L: causal attention over the whole sequence, torch's SDPA in float64
    b = 3
    L = lens[b]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[qs[b]:qs[b + 1]].transpose(1, 0, 2).astype(np.float64)),
        torch.from_numpy(np.repeat(c["kc"][b].transpose(1, 0, 2), Hq // Hkv, axis=0).astype(np.float64)),
        torch.from_numpy(np.repeat(c["vc"][b].transpose(1, 0, 2), Hq // Hkv, axis=0).astype(np.float64)),
        is_causal=True, scale=scale).numpy().transpose(1, 0, 2)
    _close(got[qs[b]:qs[b + 1]], ref, 1e-12, "causal SDPA")
    # tokens after a query's position never matter: poison them
    kp = c["k_pool"].copy()
    vp = c["v_pool"].copy()
    t_last = L - 1
    kp[c["table"][b, t_last // bs], :, t_last % bs] = 1e6
    vp[c["table"][b, t_last // bs], :, t_last % bs] = np.nan
    got2 = o.paged_attention_multi(q, kp, vp, c["table"], c["lens"], qs, scale)
    assert np.array_equal(got2[qs[b]:qs[b + 1] - 1], got[qs[b]:qs[b + 1] - 1]), "a later token leaked"
    assert np.all(np.isnan(got2[qs[b + 1] - 1])), "the last query must see the last token"


ALL_PINS = [pin_gather_roundtrip, pin_worked_example, pin_memory_formula, pin_bruteforce,
            pin_closed_forms, pin_invariants, pin_sdpa, pin_reshape_and_cache, pin_copy_blocks,
            pin_errors, pin_sliding_window, pin_multilayer_pools, pin_reblock, pin_compact_blocks,
            pin_multi_token]


# ---- 8-bit float (OCP E4M3) blocks with a scale per row: pins take oracle.fp8_cache --------

# Code -> value pairs fixed by the OCP 8-bit floating point specification (E4M3: bias 7,
# subnormals below 2^-6, largest finite 448, S.1111.111 is NaN).
_E4M3_SPEC = {0x00: 0.0, 0x01: 2.0 ** -9, 0x02: 2.0 ** -8, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
              0x0F: 1.875 * 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x70: 128.0,
              0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}


def _torch_e4m3(codes):
    """Independent decoder: torch's CPU float8_e4m3fn."""
    import torch
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_e4m3_encode(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_values(o8):
    """The value table against the specification's printed codes and torch's decoder."""
    for c, v in _E4M3_SPEC.items():
        assert o8.e4m3_value(np.uint8(c)) == v, f"code {c:#x}"
    assert np.isnan(o8.e4m3_value(np.uint8(0x7F))) and np.isnan(o8.e4m3_value(np.uint8(0xFF)))
    assert np.signbit(o8.e4m3_value(np.uint8(0x80)))
    all_codes = np.arange(256, dtype=np.uint8)
    ours, ref = o8.e4m3_value(all_codes), _torch_e4m3(all_codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert fin.sum() == 254 and np.array_equal(ours[fin], ref[fin])
    assert np.all(np.diff(ours[:0x7F]) > 0), "magnitudes must rise with the code"


def pin_e4m3_encode(o8):
    """Round trip of every finite code, ties to even at every midpoint, torch on random values."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = _torch_e4m3(codes)
    assert np.array_equal(o8.e4m3_encode(vals), codes)
    mags = _torch_e4m3(np.arange(0x7F, dtype=np.uint8))
    mid = (mags[:-1] + mags[1:]) / 2  # exact in float64
    got = o8.e4m3_encode(mid)
    lower = np.arange(0x7E)
    want = np.where(lower % 2 == 0, lower, lower + 1)
    assert np.array_equal(got, want), "midpoints must round to the even code"
    eps = (mags[1:] - mags[:-1]) / 16
    assert np.array_equal(o8.e4m3_encode(mid - eps), lower)
    assert np.array_equal(o8.e4m3_encode(mid + eps), lower + 1)
    assert np.array_equal(o8.e4m3_encode(-mid), want | 0x80)
    x = (_rng(91).uniform(-448, 448, 20000)).astype(np.float32)
    x[:100] *= np.float32(1e-3)
    assert np.array_equal(o8.e4m3_encode(x), _torch_e4m3_encode(x))


def pin_quantize_rows(o8):
    """Row quantisation: the largest magnitude maps to +-448, the dequantised row stays within
    E4M3's half-step of x, zero rows are all zero, and the codes are torch's for x / s."""
    rng = _rng(92)
    for mag in (1e-3, 1.0, 37.0, 3e4):
        x = (rng.standard_normal((6, 3, 64)) * mag).astype(np.float32)
        codes, s = o8.quantize_rows(x)
        assert codes.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (6, 3)
        imax = np.argmax(np.abs(x), axis=-1)
        top = np.take_along_axis(codes, imax[..., None], -1)[..., 0]
        assert np.all((top & 0x7F) == 0x7E), "the row maximum must take the largest code"
        deq = _torch_e4m3(codes) * s[..., None].astype(np.float64)
        bound = np.abs(x) * 2.0 ** -4 + s[..., None] * 2.0 ** -10 * 1.001 + np.abs(x) * 1e-6
        assert np.all(np.abs(deq - x) <= bound), "dequantised row outside E4M3's rounding bound"
        quot = np.clip(x / np.where(s == 0, 1, s)[..., None], -448, 448).astype(np.float32)
        assert np.array_equal(codes, _torch_e4m3_encode(quot))
    z = np.zeros((2, 8), np.float32)
    codes, s = o8.quantize_rows(z)
    assert np.all(codes == 0) and np.all(s == 0)


def _fp8_case(o8, seed, lens, Hq, Hkv, d, bs, spare=2):
    """A tiny quantised cache: random finite codes of moderate size, a random scale per row,
    unused slots holding NaN codes. Returns pools plus the per-sequence dequantised rows."""
    rng = _rng(seed, 8)
    B = len(lens)
    nbs = [-(-int(L) // bs) for L in lens]
    nb = sum(nbs) + spare
    perm = rng.permutation(nb)
    table = np.full((B, max(nbs) + 1), -1, np.int32)
    kc = np.full((nb, Hkv, bs, d), 0x7F, np.uint8)
    vc = np.full_like(kc, 0x7F)
    ks = np.full((nb, Hkv, bs), np.nan, np.float32)
    vs = np.full_like(ks, np.nan)
    rows_k, rows_v, cur = [], [], 0
    for b, L in enumerate(lens):
        ids = perm[cur:cur + nbs[b]]
        cur += nbs[b]
        table[b, :nbs[b]] = ids
        ck = rng.integers(0x20, 0x58, (L, Hkv, d)) | (rng.integers(0, 2, (L, Hkv, d)) << 7)
        cv = rng.integers(0x20, 0x58, (L, Hkv, d)) | (rng.integers(0, 2, (L, Hkv, d)) << 7)
        sk = rng.uniform(0.01, 0.2, (L, Hkv)).astype(np.float32)
        sv = rng.uniform(0.01, 0.2, (L, Hkv)).astype(np.float32)
        rk = np.zeros((L, Hkv, d))
        rv = np.zeros((L, Hkv, d))
        for t in range(L):
            for h in range(Hkv):
                kc[ids[t // bs], h, t % bs] = ck[t, h]
                vc[ids[t // bs], h, t % bs] = cv[t, h]
                ks[ids[t // bs], h, t % bs] = sk[t, h]
                vs[ids[t // bs], h, t % bs] = sv[t, h]
                rk[t, h] = _torch_e4m3(ck[t, h]) * float(sk[t, h])
                rv[t, h] = _torch_e4m3(cv[t, h]) * float(sv[t, h])
        rows_k.append(rk)
        rows_v.append(rv)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    return dict(q=q, kc=kc, vc=vc, ks=ks, vs=vs, table=table, lens=np.array(lens, np.int32),
                rows_k=rows_k, rows_v=rows_v)


def pin_fp8_decode(o8):
    """Decode over a quantised cache: brute force over rows dequantised with torch's table and
    an explicit per-row loop; K scales act like a scaled query; V scales scale the output."""
    lens, Hq, Hkv, d, bs = [1, 5, 9, 16], 4, 2, 8, 4
    c = _fp8_case(o8, 93, lens, Hq, Hkv, d, bs)
    scale = 0.3
    got = o8.paged_decode_fp8(c["q"], c["kc"], c["vc"], c["ks"], c["vs"], c["table"], c["lens"], scale)
    ref = _brute_decode(c["q"], c["rows_k"], c["rows_v"], lens, scale, Hq, Hkv)
    _close(got, ref, 1e-12, "fp8 decode vs brute force")
    k2 = o8.paged_decode_fp8(c["q"], c["kc"], c["vc"], c["ks"] * 2, c["vs"], c["table"], c["lens"], scale)
    q2 = o8.paged_decode_fp8(c["q"] * 2, c["kc"], c["vc"], c["ks"], c["vs"], c["table"], c["lens"], scale)
    assert np.array_equal(k2, q2), "doubling every K scale must equal doubling q"
    v3 = o8.paged_decode_fp8(c["q"], c["kc"], c["vc"], c["ks"], c["vs"] * 4, c["table"], c["lens"], scale)
    assert np.array_equal(v3, got * 4), "V scales must scale the output"
    for W in (1, 3, 8):
        gw = o8.paged_decode_fp8(c["q"], c["kc"], c["vc"], c["ks"], c["vs"], c["table"], c["lens"], scale,
                                 window=W)
        rw = _brute_decode(c["q"], [r[max(0, L - W):] for r, L in zip(c["rows_k"], lens)],
                           [r[max(0, L - W):] for r, L in zip(c["rows_v"], lens)],
                           [min(L, W) for L in lens], scale, Hq, Hkv)
        _close(gw, rw, 1e-12, f"fp8 window {W}")


def pin_fp8_append_and_copy(o8):
    """Quantised append lands codes and scales in the slot's block and offset (per-element
    loop), skips negative slots, and dequantises back within E4M3's bound; copy-on-write
    moves codes and scales together."""
    rng = _rng(94)
    nb, Hkv, bs, d = 6, 2, 4, 16
    kc = rng.integers(0, 256, (nb, Hkv, bs, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, Hkv, bs, d)).astype(np.uint8)
    ks = rng.uniform(0.1, 1, (nb, Hkv, bs)).astype(np.float32)
    vs = rng.uniform(0.1, 1, (nb, Hkv, bs)).astype(np.float32)
    key = rng.standard_normal((4, Hkv, d)).astype(np.float32)
    value = (rng.standard_normal((4, Hkv, d)) * 5).astype(np.float32)
    slots = np.array([5, -1, 22, 0], np.int32)
    k2, v2, ks2, vs2 = o8.reshape_and_cache_fp8(kc, vc, ks, vs, key, value, slots)
    touched = np.zeros((nb, Hkv, bs), bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = slot // bs, slot % bs
        for h in range(Hkv):
            touched[blk, h, off] = True
            for src, codes, sc in ((key, k2, ks2), (value, v2, vs2)):
                deq = _torch_e4m3(codes[blk, h, off]) * float(sc[blk, h, off])
                bound = np.abs(src[i, h]) * 2.0 ** -4 + float(sc[blk, h, off]) * 2.0 ** -10 * 1.001 + 1e-7
                assert np.all(np.abs(deq - src[i, h]) <= bound), (i, h)
    assert np.array_equal(k2[~touched], kc[~touched]) and np.array_equal(v2[~touched], vc[~touched])
    assert np.array_equal(ks2[~touched], ks[~touched]) and np.array_equal(vs2[~touched], vs[~touched])
    pairs = np.array([[2, 4], [0, 5]], np.int32)
    k3, v3, ks3, vs3 = o8.copy_blocks_fp8(kc, vc, ks, vs, pairs)
    for src, dst in pairs:
        assert np.array_equal(k3[dst], kc[src]) and np.array_equal(v3[dst], vc[src])
        assert np.array_equal(ks3[dst], ks[src]) and np.array_equal(vs3[dst], vs[src])
    assert np.array_equal(k3[[1, 3]], kc[[1, 3]]) and np.array_equal(ks3[[1, 3]], ks[[1, 3]])


FP8_PINS = [pin_e4m3_values, pin_e4m3_encode, pin_quantize_rows, pin_fp8_decode, pin_fp8_append_and_copy]
