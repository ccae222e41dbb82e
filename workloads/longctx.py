"""Seeded long-context beam workload: shared-prefix blocks, copy-on-write, one append.

Groups of beams share the physical blocks of a common prefix (reference count = beams);
each beam owns its tail blocks. The step copies the last shared block for beams 1..B-1 of
every group (the first beam keeps the original), appends one token per beam, then decodes.

Contents are drawn on the device with a seeded torch generator (the pools are gigabytes);
the layout (tables, copy pairs, slots) is plain numpy from ``default_rng([5, seed, 1])``.
Unused blocks, copy targets before the copy, and the not yet written slots of the append
blocks hold NaN. Nothing here computes attention.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

_TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class BeamWorkload:
    name: str
    dtype: str
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    scale: float
    groups: int
    beams: int
    prefix: int
    context: int
    num_blocks: int
    table_shared: np.ndarray   # int32 [B][MBS] before copy-on-write (beams share the prefix)
    table: np.ndarray          # int32 [B][MBS] after copy-on-write and with the append block
    copy_pairs: np.ndarray     # int32 [P][2]
    slot_mapping: np.ndarray   # int32 [B], the appended token of every beam
    tensors: dict              # device tensors: q, k_pool, v_pool, new_key, new_value, ...

    @property
    def batch(self) -> int:
        return self.groups * self.beams

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.table.shape[1])

    @property
    def context_lens(self) -> np.ndarray:
        return np.full(self.batch, self.context, np.int32)

    @property
    def lens_after_append(self) -> np.ndarray:
        return np.full(self.batch, self.context + 1, np.int32)

    @property
    def unique_blocks(self) -> int:
        return self.groups * (self.prefix // self.block_size) + \
            self.batch * ((self.context - self.prefix) // self.block_size)


def _randn_(t: torch.Tensor, gen: torch.Generator, chunk_rows: int = 256) -> None:
    """Fill a [N][...] tensor with N(0,1) drawn in float32 and rounded to its dtype."""
    n = t.shape[0]
    for i in range(0, n, chunk_rows):
        j = min(n, i + chunk_rows)
        t[i:j] = torch.randn(t[i:j].shape, generator=gen, device=t.device, dtype=torch.float32).to(t.dtype)


def beam_workload(device="cuda", seed: int = 0, groups: int = 8, beams: int = 4, heads: int = 32,
                  head_dim: int = 128, block_size: int = 32, prefix: int = 30720,
                  context: int = 32768, dtype: str = "bf16", spare: float = 0.10) -> BeamWorkload:
    bs = block_size
    if prefix % bs or context % bs or prefix > context:
        raise ValueError("prefix and context must be block multiples, prefix <= context")
    B = groups * beams
    nb_prefix, nb_tail = prefix // bs, (context - prefix) // bs
    needed = groups * nb_prefix + B * nb_tail + groups * (beams - 1) + B
    num_blocks = int(math.ceil(needed * (1.0 + spare)))
    rng = np.random.default_rng([5, seed, 1])
    perm = rng.permutation(num_blocks).astype(np.int32)
    cur = 0

    def take(k):
        nonlocal cur
        out = perm[cur:cur + k]
        cur += k
        return out

    mbs = nb_prefix + nb_tail + 1
    table = np.full((B, mbs), -1, np.int32)
    for grp in range(groups):
        shared = take(nb_prefix)
        for beam in range(beams):
            table[grp * beams + beam, :nb_prefix] = shared
    for b in range(B):
        table[b, nb_prefix:nb_prefix + nb_tail] = take(nb_tail)
    table_shared = table.copy()
    pairs = []
    last = nb_prefix - 1
    for grp in range(groups):
        for beam in range(1, beams):
            b = grp * beams + beam
            dst = int(take(1)[0])
            pairs.append((int(table[b, last]), dst))
            table[b, last] = dst
    append_ids = take(B)
    table[:, nb_prefix + nb_tail] = append_ids
    table_shared[:, nb_prefix + nb_tail] = append_ids
    slot_mapping = (append_ids.astype(np.int64) * bs).astype(np.int32)  # offset 0 of a fresh block

    dt = _TD[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * 5 + seed)
    shape = (num_blocks, heads, bs, head_dim)
    k_pool = torch.empty(shape, dtype=dt, device=device)
    v_pool = torch.empty(shape, dtype=dt, device=device)
    _randn_(k_pool, gen)
    _randn_(v_pool, gen)
    used = np.zeros(num_blocks, bool)
    used[table_shared[table_shared >= 0]] = True
    nan_ids = torch.from_numpy(np.nonzero(~used)[0]).to(device)  # spare blocks and copy targets
    k_pool[nan_ids] = float("nan")
    v_pool[nan_ids] = float("nan")
    aid = torch.from_numpy(append_ids.astype(np.int64)).to(device)
    k_pool[aid] = float("nan")  # the append blocks hold nothing yet
    v_pool[aid] = float("nan")
    q = torch.randn((B, heads, head_dim), generator=gen, device=device, dtype=torch.float32).to(dt)
    new_key = torch.randn((B, heads, head_dim), generator=gen, device=device, dtype=torch.float32).to(dt)
    new_value = torch.randn((B, heads, head_dim), generator=gen, device=device, dtype=torch.float32).to(dt)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)

    tensors = dict(q=q, k_pool=k_pool, v_pool=v_pool, new_key=new_key, new_value=new_value,
                   block_table=i32(table), block_table_shared=i32(table_shared),
                   context_lens=i32(np.full(B, context, np.int32)),
                   lens_after=i32(np.full(B, context + 1, np.int32)),
                   slot_mapping=i32(slot_mapping), copy_pairs=i32(np.array(pairs, np.int32).reshape(-1, 2)))
    return BeamWorkload(
        name=f"cfg5-{dtype}-beams{groups}x{beams}-L{context + 1}-prefix{prefix}-bs{bs}", dtype=dtype,
        block_size=bs, num_kv_heads=heads, num_q_heads=heads, head_dim=head_dim,
        scale=1.0 / math.sqrt(head_dim), groups=groups, beams=beams, prefix=prefix,
        context=context, num_blocks=num_blocks, table_shared=table_shared, table=table,
        copy_pairs=np.array(pairs, np.int32).reshape(-1, 2), slot_mapping=slot_mapping,
        tensors=tensors)


def host_subset(w: BeamWorkload, seqs, heads) -> dict:
    """Host (numpy float32) snapshot of what the listed sequences and heads touch in one step.

    Call it before the step runs: it copies the generator's pool contents, so nothing in it
    comes from the library. The pools hold only the blocks those sequences reference before
    or after copy-on-write (renumbered 0..n-1 in order of first use) and only the listed
    heads; tables, copy pairs and append slots are renumbered to match. Relabelling and
    selection move data only.
    """
    t = w.tensors
    seqs = list(seqs)
    heads = list(heads)
    ids, seen = [], {}
    for tab in (w.table_shared, w.table):
        for r in tab[np.asarray(seqs)]:
            for bid in r[r >= 0]:
                if int(bid) not in seen:
                    seen[int(bid)] = len(ids)
                    ids.append(int(bid))
    remap = np.full(w.num_blocks, -1, np.int64)
    remap[np.array(ids)] = np.arange(len(ids))

    def retable(tab):
        rows = tab[np.asarray(seqs)]
        return np.where(rows >= 0, remap[np.maximum(rows, 0)], -1).astype(np.int32)

    dst_of = {int(d) for d in w.copy_pairs[:, 1]}
    pairs = [(int(remap[s_]), int(remap[d])) for s_, d in w.copy_pairs.tolist()
             if d in dst_of and remap[d] >= 0]
    bs = w.block_size
    slots = np.array([remap[w.slot_mapping[b] // bs] * bs + w.slot_mapping[b] % bs for b in seqs], np.int32)
    dev = t["k_pool"].device
    hsel = torch.tensor(heads, device=dev)
    bsel = torch.tensor(ids, device=dev)
    ssel = torch.tensor(seqs, device=dev)

    def pull(x, rows):
        return x.index_select(0, rows).index_select(1, hsel).float().cpu().numpy()

    return dict(q=pull(t["q"], ssel), k_pool=pull(t["k_pool"], bsel), v_pool=pull(t["v_pool"], bsel),
                table_shared=retable(w.table_shared), table=retable(w.table),
                copy_pairs=np.array(pairs, np.int32).reshape(-1, 2), slot_mapping=slots,
                new_key=pull(t["new_key"], ssel), new_value=pull(t["new_value"], ssel),
                block_ids=np.array(ids, np.int64))
