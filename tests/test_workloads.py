"""Seeded workload generator: shapes, placement and determinism (CPU only)."""

import numpy as np

import oracle
from workloads import config_workload


def _used_ids(w, lens):
    ids = []
    for b, L in enumerate(lens):
        n = -(-int(L) // w.block_size)
        ids.extend(w.block_table[b, :n].tolist())
    return ids


def test_config1_layout():
    w = config_workload(1, seed=0)
    assert w.context_lens.tolist() == [32, 128, 64, 96]
    assert w.num_blocks == 64 and w.dtype == "f32" and w.scale == 1.0 / 8.0
    before = _used_ids(w, w.context_lens)
    after = _used_ids(w, w.lens_after_append)
    assert len(before) == 20 and len(set(before)) == 20
    assert len(after) == 24 and len(set(after)) == 24  # every length is a multiple of 16
    # the appended token lands in the new block at offset 0
    assert np.all(w.slot_mapping % 16 == 0)
    assert set((w.slot_mapping // 16).tolist()) == set(after) - set(before)
    # unwritten slots are NaN, written ones finite
    mask = np.zeros(w.k_pool.shape[:3], bool)
    for b, L in enumerate(w.context_lens):
        for t in range(L):
            mask[w.block_table[b, t // 16], :, t % 16] = True
    assert np.all(np.isfinite(w.k_pool[mask])) and np.all(np.isnan(w.k_pool[~mask]))


def test_padding_waste_reported_by_the_bench():
    """1 - sum(L) / (bs * sum(ceil(L / bs))): config 1 after its append holds 324 tokens in 24
    blocks of 16 slots (15.625% empty); contents-only lengths that fill their blocks waste
    nothing; the waste grows with the block size on the long-tail mix."""
    import bench

    w = config_workload(1, seed=0)
    assert bench.padding_waste_pct(w.context_lens, 16) == 0.0
    assert bench.padding_waste_pct(w.lens_after_append, 16) == 100.0 * (1 - 324 / 384)
    assert bench.padding_waste_pct([1], 8) == 87.5
    L = config_workload(3, seed=0, median=87).lens_after_append
    waste = [bench.padding_waste_pct(L, bs) for bs in (8, 16, 32, 64)]
    assert all(x < y for x, y in zip(waste, waste[1:]))


def test_determinism_and_block_size_independence():
    a = config_workload(3, seed=5, batch=6, heads=2, block_size=8)
    b = config_workload(3, seed=5, batch=6, heads=2, block_size=32)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.q, b.q)
    for dim in range(2):
        for s in range(6):
            ga = oracle.gather_sequence(a.k_pool, a.block_table[s], a.context_lens[s], dim)
            gb = oracle.gather_sequence(b.k_pool, b.block_table[s], b.context_lens[s], dim)
            assert np.array_equal(ga, gb)
    oa = oracle.paged_decode(a.q, a.k_pool, a.v_pool, a.block_table, a.context_lens, a.scale)
    ob = oracle.paged_decode(b.q, b.k_pool, b.v_pool, b.block_table, b.context_lens, b.scale)
    assert np.array_equal(oa, ob)
    c = config_workload(3, seed=5, batch=6, heads=2, block_size=8)
    assert np.array_equal(a.k_pool, c.k_pool, equal_nan=True)


def test_config2_lengths_and_pool():
    w = config_workload(2, seed=0, batch=64, heads=2)
    assert w.context_lens.min() >= 450 and w.context_lens.max() <= 520
    need = int(sum(-(-(int(L) + 1) // 16) for L in w.context_lens))
    assert w.num_blocks == int(np.ceil(need * 1.1))
    assert w.dtype == "f16" and w.head_dim == 128
    # values are exactly representable in fp16
    import torch
    q = torch.from_numpy(w.q)
    assert torch.equal(q.half().float(), q)


def test_append_matches_oracle_cache_op():
    w = config_workload(1, seed=3)
    k2, v2 = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    for b, L in enumerate(w.context_lens):
        g = oracle.gather_sequence(k2, w.block_table[b], L + 1, 0)
        assert np.array_equal(g[-1], w.new_key[b, 0].astype(np.float64))
        assert np.array_equal(g[:-1], oracle.gather_sequence(w.k_pool, w.block_table[b], L, 0))


def test_device_twin_matches_host_build():
    """device_paged scatters the same contents through the same tables as build_paged: its
    tensors equal build_paged(...).to_device() bit for bit (run here on the CPU device)."""
    import torch

    from workloads import build_paged, config3_lengths, device_paged, paged_contents

    lens = config3_lengths(23)[:12]
    for bs in (8, 16, 64):
        host = build_paged("t", 30, 0, lens, bs, 4, 4, 64, "f16").to_device("cpu")
        dev = device_paged("t", 30, 0, lens, bs, 4, 4, 64, "f16", "cpu").tensors
        for k in ("q", "k_pool", "v_pool", "block_table", "context_lens", "lens_after", "new_key", "new_value",
                  "slot_mapping"):
            a, b = host[k], dev[k]
            assert a.shape == b.shape and a.dtype == b.dtype, k
            if a.is_floating_point():
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), k
            else:
                assert torch.equal(a, b), k
    # shared contents across block sizes, as the sweep uses them
    c = paged_contents(30, 0, lens, 4, 4, 64, "f16")
    up: dict = {}
    a = device_paged("t", 30, 0, lens, 16, 4, 4, 64, "f16", "cpu", contents=c, uploaded=up).tensors
    b = build_paged("t", 30, 0, lens, 16, 4, 4, 64, "f16").to_device("cpu")
    assert torch.equal(a["k_pool"].view(torch.int16), b["k_pool"].view(torch.int16))


def test_contiguous_pool_is_a_relabelling():
    """The contiguous variant gives each sequence consecutive ids in order and holds the same
    tokens: the oracle's decode is bitwise that of the shuffled pool."""
    import oracle

    a = config_workload(3, median=23, block_size=16, batch=8, heads=2)
    b = config_workload(3, median=23, block_size=16, batch=8, heads=2, contiguous=True)
    assert b.name.endswith("-contiguous") and np.array_equal(a.context_lens, b.context_lens)
    nxt = 0
    for row, L in zip(b.block_table, b.lens_after_append):
        n = -(-int(L) // 16)
        assert np.array_equal(row[:n], np.arange(nxt, nxt + n)) and np.all(row[n:] == -1)
        nxt += n
    ra = oracle.paged_decode(a.q, a.k_pool, a.v_pool, a.block_table, a.context_lens, a.scale)
    rb = oracle.paged_decode(b.q, b.k_pool, b.v_pool, b.block_table, b.context_lens, b.scale)
    assert np.array_equal(ra, rb)
