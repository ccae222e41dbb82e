"""Seeded synthetic paged-KV workloads.

Every array here is a plain numpy array. Floating-point contents are drawn in float32,
rounded to the workload's storage dtype (round to nearest even, done by torch on the CPU)
and kept as float32, so the values are exactly representable in the storage dtype and the
upcast to float64 for the oracle is exact.

Layout conventions (shared by the oracle and the library):
  q                 [B][Hq][d]
  k_pool, v_pool    [num_blocks][Hkv][block_size][d]   unwritten slots hold NaN
  block_table       int32 [B][max_blocks_per_seq], -1 where unallocated
  context_lens      int32 [B], tokens already in the cache before this step's append
  new_key/new_value [B][Hkv][d], the token appended at position context_lens[b]
  slot_mapping      int32 [B], physical slot (block * block_size + offset) of that token
  copy_pairs        int32 [P][2], (src, dst) physical block ids for copy-on-write

Random streams are split so that contents do not depend on the block size or on the
physical placement: contents come from ``default_rng([cfg, seed, 0])``, the physical
permutation from ``default_rng([cfg, seed, 1, block_size])`` and the lengths from
``default_rng([cfg, seed, 2])``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def cast_like(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` (nearest even) and return them as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype]).to(torch.float32).numpy()


def lognormal_lengths(rng: np.random.Generator, n: int, median: float, sigma: float = 1.0,
                      lo: int = 4, hi: int = 4096) -> np.ndarray:
    """Long-tail lengths: round(exp(ln(median) + sigma * z)) clipped to [lo, hi]."""
    z = rng.standard_normal(n)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int32)


@dataclass
class PagedWorkload:
    name: str
    dtype: str
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    scale: float
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_table: np.ndarray
    context_lens: np.ndarray
    new_key: np.ndarray
    new_value: np.ndarray
    slot_mapping: np.ndarray
    copy_pairs: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), np.int32))
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def lens_after_append(self) -> np.ndarray:
        return (self.context_lens + 1).astype(np.int32)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPES[self.dtype]

    def to_device(self, device="cuda") -> dict:
        """Upload every array (floats in the storage dtype, ints as int32)."""
        dt = _TORCH_DTYPES[self.dtype]

        def f(x):
            # cast on the CPU first so NaN payloads match a CPU-side cast bit for bit
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dt).to(device)

        def i(x):
            return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)

        return dict(q=f(self.q), k_pool=f(self.k_pool), v_pool=f(self.v_pool),
                    block_table=i(self.block_table), context_lens=i(self.context_lens),
                    lens_after=i(self.lens_after_append), new_key=f(self.new_key),
                    new_value=f(self.new_value), slot_mapping=i(self.slot_mapping),
                    copy_pairs=i(self.copy_pairs.reshape(-1, 2)))


def _allocate_tables(rng_layout: np.random.Generator, lens: np.ndarray, bs: int,
                     num_blocks: int | None, spare: float, max_blocks_per_seq: int | None,
                     append: bool, contiguous: bool = False):
    """Hand out physical ids from one seeded permutation of the pool.

    Every sequence first receives the blocks its current tokens occupy (sequence 0 first),
    then the sequences whose append starts a new block receive one more id each, taken
    from the ids that remain. ``contiguous``: ids in order instead, each sequence's blocks
    (its append block included) consecutive, as if the cache were one dense array per
    sequence; for measuring what scattered blocks cost.
    """
    need_now = (lens + bs - 1) // bs
    need_after = (lens + (1 if append else 0) + bs - 1) // bs
    total = int(need_after.sum())
    if num_blocks is None:
        num_blocks = int(math.ceil(total * (1.0 + spare)))
    if num_blocks < total:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {total}")
    mbs = int(need_after.max()) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    perm = rng_layout.permutation(num_blocks).astype(np.int32)
    table = np.full((len(lens), mbs), -1, np.int32)
    if contiguous:
        first = np.concatenate([[0], np.cumsum(need_after)[:-1]]).astype(np.int32)
        for b, n in enumerate(need_after):
            table[b, :n] = first[b] + np.arange(n, dtype=np.int32)
        return table, num_blocks
    cur = 0
    for b, n in enumerate(need_now):
        table[b, :n] = perm[cur:cur + n]
        cur += int(n)
    for b in range(len(lens)):
        if need_after[b] > need_now[b]:
            table[b, need_now[b]] = perm[cur]
            cur += 1
    return table, num_blocks


def _scatter(pool: np.ndarray, table: np.ndarray, lens: np.ndarray, starts: np.ndarray,
             contents: np.ndarray, bs: int) -> None:
    """Write contiguous per-token rows ``contents[starts[b] + t]`` to the pool slots."""
    for b, L in enumerate(lens):
        t = np.arange(int(L))
        blk = table[b, t // bs]
        off = t % bs
        pool[blk, :, off, :] = contents[int(starts[b]) + t]


def paged_contents(cfg_id: int, seed: int, lens: np.ndarray, num_kv_heads: int, num_q_heads: int,
                   head_dim: int, dtype: str, std: float = 1.0):
    """q and the contiguous K/V rows of every sequence, independent of the block size and of
    the physical placement: (q, kc, vc, starts), sequence b's token t at row starts[b] + t
    (L + 1 rows per sequence: its cached tokens, then the token the step appends)."""
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    rng_c = np.random.default_rng([cfg_id, seed, 0])
    q = cast_like(rng_c.standard_normal((B, num_q_heads, head_dim), np.float32) * std, dtype)
    rows = int(lens.sum()) + B
    starts = np.concatenate([[0], np.cumsum(lens + 1)[:-1]]).astype(np.int64)
    kc = cast_like(rng_c.standard_normal((rows, num_kv_heads, head_dim), np.float32) * std, dtype)
    vc = cast_like(rng_c.standard_normal((rows, num_kv_heads, head_dim), np.float32) * std, dtype)
    return q, kc, vc, starts


def build_paged(name: str, cfg_id: int, seed: int, lens: np.ndarray, block_size: int,
                num_kv_heads: int, num_q_heads: int, head_dim: int, dtype: str,
                scale: float | None = None, std: float = 1.0, num_blocks: int | None = None,
                spare: float = 0.10, max_blocks_per_seq: int | None = None,
                append: bool = True, contents=None, contiguous: bool = False) -> PagedWorkload:
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    rng_l = np.random.default_rng([cfg_id, seed, 1, block_size])
    table, nb = _allocate_tables(rng_l, lens, block_size, num_blocks, spare,
                                 max_blocks_per_seq, append, contiguous)
    # Contents: q, then L+1 contiguous K rows per sequence, then the same for V.
    if contents is None:
        contents = paged_contents(cfg_id, seed, lens, num_kv_heads, num_q_heads, head_dim, dtype, std)
    q, kc, vc, starts = contents
    k_pool = np.full((nb, num_kv_heads, block_size, head_dim), np.nan, np.float32)
    v_pool = np.full_like(k_pool, np.nan)
    _scatter(k_pool, table, lens, starts, kc, block_size)
    _scatter(v_pool, table, lens, starts, vc, block_size)
    new_key = kc[starts + lens]
    new_value = vc[starts + lens]
    if append:
        slot = table[np.arange(B), lens // block_size].astype(np.int64) * block_size + lens % block_size
        slot_mapping = slot.astype(np.int32)
    else:
        slot_mapping = np.full(B, -1, np.int32)
    return PagedWorkload(
        name=name, dtype=dtype, block_size=block_size, num_kv_heads=num_kv_heads,
        num_q_heads=num_q_heads, head_dim=head_dim, scale=float(scale), q=q,
        k_pool=k_pool, v_pool=v_pool, block_table=table, context_lens=lens,
        new_key=new_key, new_value=new_value, slot_mapping=slot_mapping,
        meta={"cfg": cfg_id, "seed": seed, "std": std,
              "contents_k": kc, "contents_v": vc, "starts": starts},
    )


def config_workload(cfg: int, seed: int = 0, *, block_size: int | None = None,
                    median: float | None = None, batch: int | None = None,
                    heads: int | None = None, sigma: float = 1.0,
                    contiguous: bool = False) -> PagedWorkload:
    """The five seeded synthetic workloads (configs 1-4 here; 5 lives in ``longctx``).

    ``batch``/``heads`` shrink a configuration for quick tests while keeping its dtype,
    head_dim, block size and length distribution. ``contiguous`` places each sequence's
    blocks consecutively in id order (same lengths and contents; name suffix -contiguous).
    """
    rng_len = np.random.default_rng([cfg, seed, 2])
    if cfg == 1:
        lens = np.array([32, 128, 64, 96], np.int32)
        return build_paged("cfg1-f32-tiny", 1, seed, lens, block_size or 16, heads or 8,
                           heads or 8, 64, "f32", scale=1.0 / 8.0, num_blocks=64)
    if cfg == 2:
        B = batch or 64
        H = heads or 32
        lens = rng_len.integers(450, 521, size=64).astype(np.int32)[:B]
        return build_paged("cfg2-f16-mha" + ("-contiguous" if contiguous else ""), 2, seed, lens,
                           block_size or 16, H, H, 128, "f16", std=0.5, contiguous=contiguous)
    if cfg == 3:
        B = batch or 256
        H = heads or 32
        med = median or 87
        lens = lognormal_lengths(rng_len, 256, med, sigma)[:B]
        bs = block_size or 16
        return build_paged(f"cfg3-f16-longtail-med{med:g}-bs{bs}" + ("-contiguous" if contiguous else ""),
                           3 if med == 87 else 30, seed, lens, bs, H, H, 128, "f16", contiguous=contiguous)
    if cfg == 4:
        B = batch or 32
        hkv = heads or 8
        lens = np.full(B, 2048, np.int32)
        bs = block_size or 16
        return build_paged(f"cfg4-bf16-gqa-bs{bs}" + ("-contiguous" if contiguous else ""), 4, seed, lens, bs,
                           hkv, hkv * 8, 128, "bf16", contiguous=contiguous)
    raise ValueError(f"unknown config {cfg}")


@dataclass
class DevicePagedWorkload:
    """The device tensors of ``build_paged(...).to_device()`` built without the host pools: the
    contents are drawn on the host by the same generator, uploaded once and scattered through
    the tables on the device (for timing runs at full size; the oracle needs PagedWorkload)."""
    name: str
    dtype: str
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    scale: float
    num_blocks: int
    block_table: np.ndarray
    context_lens: np.ndarray
    slot_mapping: np.ndarray
    tensors: dict

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def lens_after_append(self) -> np.ndarray:
        return (self.context_lens + 1).astype(np.int32)


def device_paged(name: str, cfg_id: int, seed: int, lens: np.ndarray, block_size: int, num_kv_heads: int,
                 num_q_heads: int, head_dim: int, dtype: str, device, scale: float | None = None,
                 std: float = 1.0, spare: float = 0.10, contents=None, uploaded=None) -> DevicePagedWorkload:
    """Device twin of build_paged (append=True, default pool size): the same tables, slots and
    values bit for bit. ``contents`` (from paged_contents) and ``uploaded`` (their device
    copies, a dict filled on first use) may be shared by several block sizes."""
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    bs = block_size
    rng_l = np.random.default_rng([cfg_id, seed, 1, bs])
    table, nb = _allocate_tables(rng_l, lens, bs, None, spare, None, True)
    if contents is None:
        contents = paged_contents(cfg_id, seed, lens, num_kv_heads, num_q_heads, head_dim, dtype, std)
    q, kc, vc, starts = contents
    dt = _TORCH_DTYPES[dtype]
    up = {} if uploaded is None else uploaded
    if not up:
        for key, x in (("q", q), ("kc", kc), ("vc", vc)):
            up[key] = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dt).to(device)
    seq = np.repeat(np.arange(B), lens)
    tok = np.arange(int(lens.sum())) - np.repeat(np.cumsum(lens) - lens, lens)
    blk = torch.from_numpy(table[seq, tok // bs].astype(np.int64)).to(device)
    off = torch.from_numpy((tok % bs).astype(np.int64)).to(device)
    rows = torch.from_numpy((starts[seq] + tok).astype(np.int64)).to(device)
    pools = []
    for src in (up["kc"], up["vc"]):
        pool = torch.full((nb, num_kv_heads, bs, head_dim), float("nan"), dtype=dt, device=device)
        pool[blk, :, off, :] = src.index_select(0, rows)
        pools.append(pool)
    new_rows = torch.from_numpy((starts + lens).astype(np.int64)).to(device)
    slot = (table[np.arange(B), lens // bs].astype(np.int64) * bs + lens % bs).astype(np.int32)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)

    tensors = dict(q=up["q"], k_pool=pools[0], v_pool=pools[1], block_table=i32(table), context_lens=i32(lens),
                   lens_after=i32(lens + 1), new_key=up["kc"].index_select(0, new_rows),
                   new_value=up["vc"].index_select(0, new_rows), slot_mapping=i32(slot),
                   copy_pairs=i32(np.zeros((0, 2), np.int32)))
    return DevicePagedWorkload(name=name, dtype=dtype, block_size=bs, num_kv_heads=num_kv_heads,
                               num_q_heads=num_q_heads, head_dim=head_dim, scale=float(scale), num_blocks=nb,
                               block_table=table, context_lens=lens, slot_mapping=slot, tensors=tensors)


def config3_lengths(median: float, seed: int = 0, sigma: float = 1.0, batch: int = 256) -> np.ndarray:
    """The long-tail lengths of the block-size sweep (cached tokens before the step)."""
    return lognormal_lengths(np.random.default_rng([3, seed, 2]), 256, median, sigma)[:batch]


def config3_device_family(median: float, block_sizes, device, seed: int = 0):
    """The block-size sweep at one median, on the device: one DevicePagedWorkload per block
    size, all with the same contents (they equal config_workload(3, median=..., block_size=...)
    uploaded)."""
    lens = config3_lengths(median, seed)
    cfg_id = 3 if median == 87 else 30
    contents = paged_contents(cfg_id, seed, lens, 32, 32, 128, "f16")
    up: dict = {}
    out = []
    for bs in block_sizes:
        out.append(device_paged(f"cfg3-f16-longtail-med{median:g}-bs{bs}", cfg_id, seed, lens, bs, 32, 32, 128,
                                "f16", device, contents=contents, uploaded=up))
    return out
