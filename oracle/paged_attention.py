"""Plain float64 reference for paged-KV decode attention and the cache operations.

Test infrastructure only: imported by tests/, the smoke check and the CPU-baseline leg of
bench.py, never by the library.

Pages cited (each by title and section):
  [BlockManager essay]  "KV Cache & BlockManager", dpshk.com/news/5906718
  [KV Block course]     vLLM memory management course, ch. 3 "KV Block design"
  [Valid-length essay]  KV cache valid-length / padding-KV bug, dpshk.com/news/5937191
  [CANN paging article] "KV Cache paging optimisation in LLM inference", intelliparadigm.com

What is computed (readings of points the pages leave open are listed in the design notes):
  * A sequence's logical block j lives in physical block block_table[b][j]; token t sits at
    offset t % block_size inside it ([BlockManager essay] §2; [KV Block course] §3.3).
  * Each block holds [kv_heads][block_size][head_dim] for K and the same for V
    ([BlockManager essay] §5.1; [KV Block course] §3.2).
  * Only the first context_len tokens are valid; padding is never used
    ([Valid-length essay] §2.4, §4.1, §4.2).
  * The decode query dots with every earlier key, softmax, weighted sum of values
    ([Valid-length essay] §3.1; [CANN paging article] §2.2). Paging changes where K/V
    live, not the result, so the oracle gathers the blocks back into contiguous K/V and
    evaluates the plain definition in float64.
  * Grouped-query heads: query head h reads kv head h // (Hq / Hkv) (a reading; the
    pages only speak of num_heads).

Parity pins for every function here live in tests/test_oracle_pins.py.
"""

from __future__ import annotations

import numpy as np


class OracleInputError(ValueError):
    """Raised where the library would flag a device error (bad id, bad length, bad slot)."""


def blocks_needed(context_len: int, block_size: int) -> int:
    """Number of blocks a sequence of ``context_len`` tokens occupies: ceil(L / bs).

    [BlockManager essay] §2: 128 tokens in 16-token blocks occupy 8 blocks.
    """
    return -(-int(context_len) // int(block_size))


def kv_cache_bytes(num_kv_heads: int, head_dim: int, dtype_bytes: int, context_lens,
                   num_layers: int = 1) -> int:
    """Bytes of valid K and V: 2 x layers x kv_heads x sum(tokens) x head_dim x dtype_bytes.

    [BlockManager essay] §1 tip (memory formula) and [KV Block course] §3.2. The batch
    enters only through the sum of the per-sequence token counts.
    """
    total_tokens = int(np.sum(np.asarray(context_lens, dtype=np.int64)))
    return 2 * int(num_layers) * int(num_kv_heads) * total_tokens * int(head_dim) * int(dtype_bytes)


def allocated_kv_bytes(num_kv_heads: int, head_dim: int, dtype_bytes: int, context_lens,
                       block_size: int, num_layers: int = 1) -> int:
    """Bytes of whole blocks held: as ``kv_cache_bytes`` with each length rounded up to blocks."""
    nb = sum(blocks_needed(L, block_size) for L in np.asarray(context_lens).tolist())
    return 2 * int(num_layers) * int(num_kv_heads) * nb * int(block_size) * int(head_dim) * int(dtype_bytes)


def gather_range(pool: np.ndarray, table_row: np.ndarray, start: int, stop: int, kv_head: int) -> np.ndarray:
    """Contiguous float64 rows [start, stop) of one sequence and kv head.

    Walks the logical blocks that hold those tokens in order, reads physical block
    table_row[j] ([BlockManager essay] §2, §5.2; [KV Block course] §3.3), concatenates the
    per-block [block_size][head_dim] slabs and keeps exactly the requested rows. Blocks
    outside the range are never read, so padding, unallocated entries and blocks released
    before a window are never touched ([Valid-length essay] §4.1).
    """
    num_blocks, _, block_size, _ = pool.shape
    start, stop = int(start), int(stop)
    if stop <= 0:
        raise OracleInputError(f"context_len {stop} <= 0")
    if not 0 <= start < stop:
        raise OracleInputError(f"empty token range [{start}, {stop})")
    nb = blocks_needed(stop, block_size)
    if nb > len(table_row):
        raise OracleInputError(f"context_len {stop} needs {nb} blocks > table width {len(table_row)}")
    j0 = start // block_size
    slabs = []
    for j in range(j0, nb):
        pid = int(table_row[j])
        if not 0 <= pid < num_blocks:
            raise OracleInputError(f"block id {pid} at logical block {j} outside [0, {num_blocks})")
        slabs.append(pool[pid, kv_head])
    rows = np.concatenate(slabs, axis=0)
    return rows[start - j0 * block_size: stop - j0 * block_size].astype(np.float64)


def gather_sequence(pool: np.ndarray, table_row: np.ndarray, context_len: int, kv_head: int) -> np.ndarray:
    """Contiguous [context_len][head_dim] float64 rows of one sequence and kv head (all its tokens)."""
    return gather_range(pool, table_row, 0, context_len, kv_head)


def attention_one_query(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query over L keys, in float64.

    [Valid-length essay] §3.1: the new token's query dots with every earlier key and the
    values are summed with those weights; [CANN paging article] §2.2 steps 2-4.
    """
    s = float(scale) * (K @ q.astype(np.float64))
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def paged_decode_heads(q, k_pool, v_pool, block_table, context_lens, scale, pairs):
    """Decode output for the listed (sequence, query head) pairs only: float64 [n][d]."""
    Hq = q.shape[1]
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise OracleInputError(f"num_q_heads {Hq} not a multiple of num_kv_heads {Hkv}")
    group = Hq // Hkv
    out = np.empty((len(pairs), q.shape[2]), np.float64)
    for i, (b, h) in enumerate(pairs):
        g = h // group
        K = gather_sequence(k_pool, block_table[b], context_lens[b], g)
        V = gather_sequence(v_pool, block_table[b], context_lens[b], g)
        out[i] = attention_one_query(q[b, h], K, V, scale)
    return out


def paged_decode(q, k_pool, v_pool, block_table, context_lens, scale) -> np.ndarray:
    """Single-query decode attention over a paged cache: float64 [B][Hq][d].

    For sequence b and query head h: gather K and V of kv head h // (Hq/Hkv) through the
    block table, then take the plain softmax attention of q[b][h] over those L rows.
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise OracleInputError(f"num_q_heads {Hq} not a multiple of num_kv_heads {Hkv}")
    group = Hq // Hkv
    out = np.empty((B, Hq, d), np.float64)
    for b in range(B):
        for g in range(Hkv):
            K = gather_sequence(k_pool, block_table[b], context_lens[b], g)
            V = gather_sequence(v_pool, block_table[b], context_lens[b], g)
            for h in range(g * group, (g + 1) * group):
                out[b, h] = attention_one_query(q[b, h], K, V, scale)
    return out


def window_start(context_len: int, window: int) -> int:
    """First attended token of a sliding window of the last ``window`` tokens.

    [Valid-length essay] §3.3 and §5.3: the sliding-window policy keeps only the most recent
    N tokens' K/V.
    """
    return max(0, int(context_len) - int(window))


def paged_decode_window(q, k_pool, v_pool, block_table, context_lens, scale, window) -> np.ndarray:
    """Decode over the last ``window`` tokens of every sequence: float64 [B][Hq][d]."""
    if int(window) <= 0:
        raise OracleInputError("window must be positive")
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise OracleInputError(f"num_q_heads {Hq} not a multiple of num_kv_heads {Hkv}")
    group = Hq // Hkv
    out = np.empty((B, Hq, d), np.float64)
    for b in range(B):
        L = int(context_lens[b])
        lo = window_start(L, window)
        for g in range(Hkv):
            K = gather_range(k_pool, block_table[b], lo, L, g)
            V = gather_range(v_pool, block_table[b], lo, L, g)
            for h in range(g * group, (g + 1) * group):
                out[b, h] = attention_one_query(q[b, h], K, V, scale)
    return out


def reshape_and_cache(k_pool, v_pool, key, value, slot_mapping):
    """Append new tokens' K/V into their pool slots; returns updated copies of the pools.

    Token i (rows key[i], value[i] of shape [kv_heads][head_dim]) goes to physical block
    slot // block_size at offset slot % block_size, for every kv head, so a block's
    physical token order equals its logical order ([BlockManager essay] §4.4;
    [Valid-length essay] §4.1: writes land at the valid length). A negative slot marks a
    padding token and is skipped: padding KV never enters the cache ([Valid-length essay]
    §2.3). A slot beyond the pool raises.
    """
    k_new = k_pool.copy()
    v_new = v_pool.copy()
    num_blocks, _, block_size, _ = k_pool.shape
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        if blk >= num_blocks:
            raise OracleInputError(f"slot {slot} outside a pool of {num_blocks} x {block_size}")
        k_new[blk, :, off, :] = key[i]
        v_new[blk, :, off, :] = value[i]
    return k_new, v_new


def copy_blocks(k_pool, v_pool, pairs):
    """Copy-on-write: physical block dst becomes a copy of src, for K and V, every head.

    [BlockManager essay] §2 and §4.2, [KV Block course] §3.4: a block shared by several
    sequences (e.g. beams) carries a reference count; a sharer that must diverge gets its
    own copy. Pairs are applied in order; an id outside the pool or src == dst raises.
    """
    k_new = k_pool.copy()
    v_new = v_pool.copy()
    num_blocks = k_pool.shape[0]
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks) or src == dst:
            raise OracleInputError(f"bad copy pair ({src}, {dst}) for a pool of {num_blocks}")
        k_new[dst] = k_new[src]
        v_new[dst] = v_new[src]
    return k_new, v_new


def layer_pools(cache: np.ndarray, layer: int):
    """K and V pools of one layer of a multi-layer cache [num_blocks][2][num_layers][heads]
    [block_size][head_dim], whose dim 1 selects K or V ([BlockManager essay] §5.1). The views
    share the cache's memory; consecutive blocks are 2 * num_layers slabs apart."""
    return cache[:, 0, int(layer)], cache[:, 1, int(layer)]


def reblock(pool, block_table, context_lens, new_block_size: int, new_table, new_num_blocks: int):
    """Migrate a paged cache to another block size ([CANN paging article] §4.1: a new block
    size invalidates the tables, so the block contents move to a new layout).

    Every sequence's valid rows, read through its old table, are written in order into the
    blocks its new table lists, block_size ``new_block_size`` each. Returns the new pool;
    slots that hold no valid token are NaN. Bad ids or lengths raise.
    """
    nb_old, H, bs, d = pool.shape
    out = np.full((int(new_num_blocks), H, int(new_block_size), d), np.nan, pool.dtype)
    nbs = int(new_block_size)
    for b, L in enumerate(np.asarray(context_lens).tolist()):
        need = blocks_needed(L, nbs)
        if need > np.shape(new_table)[1]:
            raise OracleInputError(f"sequence {b}: {need} new blocks > new table width")
        for h in range(H):
            rows = gather_sequence(pool, block_table[b], L, h)
            for j in range(need):
                pid = int(new_table[b][j])
                if not 0 <= pid < new_num_blocks:
                    raise OracleInputError(f"new block id {pid} outside [0, {new_num_blocks})")
                chunk = rows[j * nbs:(j + 1) * nbs]
                out[pid, h, :len(chunk)] = chunk
    return out


def compact_blocks(k_pool, v_pool, block_table, pairs):
    """Defragmentation step ([CANN paging article] §5.1): live blocks move to their new ids
    (copy-on-write's block copy, pair by pair) and every table entry naming a moved block is
    rewritten to its new id. Returns (k_pool, v_pool, block_table)."""
    k_new, v_new = copy_blocks(k_pool, v_pool, pairs)
    moved = {int(s): int(d) for s, d in np.asarray(pairs).reshape(-1, 2).tolist()}
    table = np.array(block_table, copy=True)
    for idx, pid in np.ndenumerate(table):
        if int(pid) in moved:
            table[idx] = moved[int(pid)]
    return k_new, v_new, table


def paged_attention_multi(q, k_pool, v_pool, block_table, context_lens, query_start, scale) -> np.ndarray:
    """Several new query tokens per sequence over a paged cache, causally masked: float64
    [num_q_tokens][Hq][d].

    Sequence b owns query rows query_start[b] .. query_start[b+1]-1 (n_b tokens). Its cache
    already holds those tokens, appended after the history, so its length L_b includes them
    ([Valid-length essay] §2.2: each round's tokens are appended after the previous rounds').
    Query i sits at position p = L_b - n_b + i and attends to tokens 0 .. p only: the causal
    mask inside the valid range ([Valid-length essay] §4.2, key j visible to query i iff
    j <= i). n_b = 1 is the single-query decode.
    """
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise OracleInputError(f"num_q_heads {Hq} not a multiple of num_kv_heads {Hkv}")
    group = Hq // Hkv
    qs = np.asarray(query_start, np.int64)
    if qs[0] != 0 or qs[-1] != T or np.any(np.diff(qs) < 0):
        raise OracleInputError("query_start must rise from 0 to the number of query rows")
    out = np.full((T, Hq, d), np.nan, np.float64)
    for b, L in enumerate(np.asarray(context_lens).tolist()):
        n = int(qs[b + 1] - qs[b])
        if n > L:
            raise OracleInputError(f"sequence {b}: {n} new tokens > context length {L}")
        if n == 0:
            continue
        for g in range(Hkv):
            K = gather_sequence(k_pool, block_table[b], L, g)
            V = gather_sequence(v_pool, block_table[b], L, g)
            for i in range(n):
                p = L - n + i
                for h in range(g * group, (g + 1) * group):
                    out[qs[b] + i, h] = attention_one_query(q[qs[b] + i, h], K[:p + 1], V[:p + 1], scale)
    return out
