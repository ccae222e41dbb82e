"""Host block manager: allocation, reference counts, copy-on-write, rejection (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle
from paged_kv_cache_indexed_amd.block_manager import BlockManager, BlockTableOverflow, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fill(bm, sid, n):
    slots, pairs = bm.append_slots(sid, n)
    return slots, pairs


def test_worked_example_tables():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_blockmanager_s2.json")))
    bm = BlockManager(num_blocks=100, block_size=g["block_size"], max_blocks_per_seq=10, shuffle_seed=3)
    ids = list(range(4))
    for sid, L in zip(ids, g["context_lens"]):
        bm.add_sequence(sid)
        _fill(bm, sid, L)
    t = bm.block_table(ids)
    counts = [(row >= 0).sum() for row in t]
    assert counts == [2, 8, 4, 6] and sum(counts) == 20
    used = t[t >= 0]
    assert len(set(used.tolist())) == 20  # no physical block is shared
    assert bm.context_lens(ids).tolist() == g["context_lens"]
    assert bm.num_free == 80
    bm.check_invariants()


def test_slots_follow_the_table():
    bm = BlockManager(64, 16, 8, shuffle_seed=1)
    bm.add_sequence(0)
    slots, _ = bm.append_slots(0, 37)
    row = bm.block_table([0])[0]
    for t, s in enumerate(slots):
        assert s // 16 == row[t // 16] and s % 16 == t % 16


def test_overflow_is_rejected_without_side_effects():
    # [BlockManager essay] section 4.1: max_model_len 2048 at block size 16 (128 blocks),
    # a 2050-token request needs 129 blocks.
    bm = BlockManager(num_blocks=1000, block_size=16, max_blocks_per_seq=128)
    bm.add_sequence(0)
    before = bm.num_free
    with pytest.raises(BlockTableOverflow):
        bm.append_slots(0, 2050)
    assert bm.num_free == before and bm.length(0) == 0
    bm.append_slots(0, 2048)
    with pytest.raises(BlockTableOverflow):
        bm.append_slots(0, 1)
    bm.check_invariants()


def test_exhaustion_raises():
    bm = BlockManager(num_blocks=3, block_size=8, max_blocks_per_seq=10)
    bm.add_sequence(0)
    bm.append_slots(0, 24)
    with pytest.raises(OutOfBlocks, match="Out of GPU blocks"):
        bm.append_slots(0, 1)
    assert bm.length(0) == 24
    bm.check_invariants()


def test_cancel_releases_every_reference():
    # [BlockManager essay] section 4.2: a cancelled request must not leak its blocks.
    bm = BlockManager(num_blocks=50, block_size=16, max_blocks_per_seq=10)
    for i in range(20):
        try:
            with bm.sequence(100 + i) as sid:
                bm.append_slots(sid, 40)
                if i % 3 == 0:
                    raise TimeoutError("cancelled")
        except TimeoutError:
            pass
    assert bm.num_free == 50 and int(bm.ref_count.sum()) == 0
    bm.check_invariants()


def test_double_free_raises():
    bm = BlockManager(4, 8, 4)
    b = bm.allocate_block()
    bm.release_block(b)
    with pytest.raises(ValueError):
        bm.release_block(b)


def test_fork_and_copy_on_write():
    bm = BlockManager(num_blocks=40, block_size=16, max_blocks_per_seq=8, shuffle_seed=0)
    bm.add_sequence(0)
    bm.append_slots(0, 20)  # 2 blocks, the second partly filled
    for c in (1, 2, 3):
        bm.fork(0, c)
    last = bm.blocks(0)[1]
    assert bm.ref_count[last] == 4 and bm.ref_count[bm.blocks(0)[0]] == 4
    pairs = []
    for c in (1, 2, 3):
        slots, p = bm.append_slots(c, 1)
        assert len(p) == 1 and p[0][0] == last
        assert slots[0] // 16 == p[0][1] and slots[0] % 16 == 4
        pairs += p
    # the forking sequence keeps the original and writes in place
    slots, p = bm.append_slots(0, 1)
    assert p == [] and slots[0] // 16 == last
    assert len({d for _, d in pairs}) == 3 and bm.ref_count[last] == 1
    assert bm.ref_count[bm.blocks(0)[0]] == 4  # the full first block stays shared
    bm.check_invariants()
    for s in (0, 1, 2, 3):
        bm.free_sequence(s)
    assert bm.num_free == 40
    bm.check_invariants()


def test_shared_prefix_layout_like_the_beam_workload():
    # 2 groups x 4 beams, a prefix ending on a block boundary, private tails, then a
    # copy-on-write of the last shared block for beams 1..3 of each group.
    bs, prefix, tail = 8, 40, 16
    bm = BlockManager(num_blocks=64, block_size=bs, max_blocks_per_seq=16, shuffle_seed=5)
    seqs = []
    for grp in range(2):
        root = 4 * grp
        bm.add_sequence(root)
        bm.append_slots(root, prefix)
        for beam in range(1, 4):
            bm.fork(root, root + beam)
        for beam in range(4):
            _, p = bm.append_slots(root + beam, tail)
            assert p == []  # the prefix ended on a block boundary
        seqs += [root + k for k in range(4)]
    unique = 2 * prefix // bs + 8 * tail // bs
    assert bm.num_blocks - bm.num_free == unique
    pairs = [bm.copy_on_write(s, prefix // bs - 1) for s in seqs if s % 4 != 0]
    assert len(pairs) == 6 and all(p is not None for p in pairs)
    t = bm.block_table(seqs)
    for grp in range(2):
        rows = t[4 * grp:4 * grp + 4]
        assert all((rows[k, :prefix // bs - 1] == rows[0, :prefix // bs - 1]).all() for k in range(4))
        assert len(set(rows[:, prefix // bs - 1].tolist())) == 4
    bm.check_invariants()


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(11)
    bm = BlockManager(num_blocks=200, block_size=8, max_blocks_per_seq=30, shuffle_seed=2)
    live = []
    nxt = 0
    for _ in range(600):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                bm.add_sequence(nxt)
                live.append(nxt)
                nxt += 1
            elif op == 1:
                bm.append_slots(live[rng.integers(len(live))], int(rng.integers(1, 20)))
            elif op == 2:
                bm.fork(live[rng.integers(len(live))], nxt)
                live.append(nxt)
                nxt += 1
            else:
                bm.free_sequence(live.pop(rng.integers(len(live))))
        except (OutOfBlocks, BlockTableOverflow):
            pass
        bm.check_invariants()


def test_manager_slots_drive_the_oracle_cache():
    # Paging round trip: tokens appended through the manager's slots and the oracle's
    # reshape_and_cache gather back to the contiguous contents.
    rng = np.random.default_rng(4)
    bs, H, d = 4, 2, 3
    bm = BlockManager(num_blocks=30, block_size=bs, max_blocks_per_seq=10, shuffle_seed=9)
    kp = np.full((30, H, bs, d), np.nan, np.float32)
    vp = kp.copy()
    contents = {}
    for sid, L in ((0, 11), (1, 4), (2, 1)):
        bm.add_sequence(sid)
        k = rng.standard_normal((L, H, d)).astype(np.float32)
        slots, _ = bm.append_slots(sid, L)
        kp, vp = oracle.reshape_and_cache(kp, vp, k, k, slots)
        contents[sid] = k
    t = bm.block_table([0, 1, 2])
    for r, sid in enumerate((0, 1, 2)):
        for h in range(H):
            got = oracle.gather_sequence(kp, t[r], bm.length(sid), h)
            assert np.array_equal(got, contents[sid][:, h].astype(np.float64))


def _fragmented(seed=0, nb=64, bs=4):
    rng = np.random.default_rng(seed)
    bm = BlockManager(nb, bs, 16, shuffle_seed=seed)
    for sid in range(10):
        bm.add_sequence(sid)
        bm.append_slots(sid, int(rng.integers(1, 20)))
    bm.fork(2, 100)  # shared blocks move as one
    bm.append_slots(100, 3)
    for sid in (1, 4, 7):
        bm.free_sequence(sid)
    return bm


def test_compact_moves_live_blocks_to_the_front_and_keeps_contents():
    import oracle

    bm = _fragmented()
    seqs = sorted(bm._seqs)
    before = bm.block_table(seqs)
    lens = bm.context_lens(seqs)
    assert not bm.is_compact()
    rng = np.random.default_rng(1)
    pool_k = rng.standard_normal((bm.num_blocks, 2, bm.block_size, 3))
    pool_v = rng.standard_normal((bm.num_blocks, 2, bm.block_size, 3))
    live_before = set(np.nonzero(bm.ref_count)[0].tolist())
    pairs = bm.compact()
    bm.check_invariants()
    assert bm.is_compact()
    assert {int(s) for s in pairs[:, 0]} <= live_before
    assert not ({int(d) for d in pairs[:, 1]} & live_before), "a destination must be free"
    after = bm.block_table(seqs)
    k2, v2, t2 = oracle.compact_blocks(pool_k, pool_v, before, pairs)
    assert np.array_equal(t2, after), "the planner's tables must equal the relabelled tables"
    for r, L in enumerate(lens):
        for h in range(2):
            assert np.array_equal(oracle.gather_sequence(k2, after[r], L, h),
                                  oracle.gather_sequence(pool_k, before[r], L, h))
    assert bm.allocate_block() == bm.num_live() - 1  # the lowest free id comes next
    assert len(bm.compact()) == 0 or bm.is_compact()


def test_reblocked_manager_holds_the_same_sequences():
    bm = _fragmented(3)
    seqs = sorted(bm._seqs)
    for bs in (1, 2, 8, 32):
        nb2 = bm.reblocked(bs)
        nb2.check_invariants()
        assert np.array_equal(nb2.context_lens(seqs), bm.context_lens(seqs))
        t = nb2.block_table(seqs)
        for r, L in enumerate(bm.context_lens(seqs)):
            n = -(-int(L) // bs)
            assert np.all(t[r, :n] >= 0) and np.all(t[r, n:] == -1)
