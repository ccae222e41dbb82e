"""Torch-facing helpers over the C ABI: allocate outputs and workspaces, then call the library.

Allocation is torch's; every arithmetic step runs in libpagedkv's HIP kernels.
"""

from __future__ import annotations

import torch

from ._lib import (CacheDesc, pa_copy_blocks, pa_copy_blocks_fp8, pa_decode, pa_decode_append, pa_decode_append_fp8,
                   pa_decode_beams, pa_decode_beams_workspace_bytes,
                   pa_decode_fp8, pa_decode_sliding_window, pa_decode_sliding_window_workspace_bytes,
                   pa_decode_workspace_bytes, pa_multi_token_attention, pa_multi_token_workspace_bytes,
                   pa_reblock, pa_reshape_and_cache, pa_reshape_and_cache_fp8)


def workspace_for(k_pool: torch.Tensor, batch: int, num_q_heads: int, max_context_len: int,
                  partition_size: int = 0, window: int = 0):
    """A float32 workspace tensor of the size the decode needs, or None if it needs none."""
    if window > 0:
        n = pa_decode_sliding_window_workspace_bytes(CacheDesc.of(k_pool), batch, num_q_heads,
                                                     max_context_len, window, partition_size)
    else:
        n = pa_decode_workspace_bytes(CacheDesc.of(k_pool), batch, num_q_heads, max_context_len,
                                      partition_size)
    if n == 0:
        return None
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=k_pool.device)


def decode(q, k_pool, v_pool, block_table, context_lens, max_context_len: int, scale: float,
           partition_size: int = 0, out=None, workspace=None, err_flag=None, stream=None,
           window: int = 0):
    """Paged decode attention; returns ``out`` [batch][num_q_heads][head_dim] in q's dtype.

    ``window`` > 0 attends to the last ``window`` tokens of each sequence only."""
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = workspace_for(k_pool, q.shape[0], q.shape[1], max_context_len, partition_size,
                                  window)
    if window > 0:
        pa_decode_sliding_window(CacheDesc.of(k_pool), out, q, k_pool, v_pool, block_table, context_lens,
                                 max_context_len, scale, window, partition_size, workspace, err_flag,
                                 stream)
    else:
        pa_decode(CacheDesc.of(k_pool), out, q, k_pool, v_pool, block_table, context_lens,
                  max_context_len, scale, partition_size, workspace, err_flag, stream)
    return out


def decode_append(q, k_pool, v_pool, block_table, context_lens, max_context_len: int, scale: float, key, value,
                  slot_mapping, partition_size: int = 0, out=None, workspace=None, err_flag=None, stream=None):
    """reshape_and_cache of one token per sequence, then decode over the grown contexts
    (context_lens include the new token), in one launch."""
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = workspace_for(k_pool, q.shape[0], q.shape[1], max_context_len, partition_size)
    pa_decode_append(CacheDesc.of(k_pool), out, q, k_pool, v_pool, block_table, context_lens, max_context_len,
                     scale, key, value, slot_mapping, partition_size, workspace, err_flag, stream)
    return out


def reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, err_flag=None, stream=None):
    pa_reshape_and_cache(CacheDesc.of(k_pool), key, value, k_pool, v_pool, slot_mapping, err_flag,
                         stream)


def copy_blocks(k_pool, v_pool, pairs, err_flag=None, stream=None):
    pa_copy_blocks(CacheDesc.of(k_pool), k_pool, v_pool, pairs, err_flag, stream)


# ---- 8-bit float (OCP E4M3) pools: uint8 codes plus a float32 scale per (block, head, offset)

def empty_fp8_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, device):
    """Uninitialised (k_pool, v_pool, k_scale, v_scale) for an 8-bit float cache."""
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    return (torch.empty(shape, dtype=torch.uint8, device=device),
            torch.empty(shape, dtype=torch.uint8, device=device),
            torch.empty(shape[:3], dtype=torch.float32, device=device),
            torch.empty(shape[:3], dtype=torch.float32, device=device))


def decode_fp8(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, max_context_len: int,
               scale: float, window: int = 0, partition_size: int = 0, out=None, workspace=None,
               err_flag=None, stream=None):
    """Decode over an 8-bit float cache; ``out`` has q's dtype (fp16 or bf16)."""
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = workspace_for(k_pool, q.shape[0], q.shape[1], max_context_len, partition_size,
                                  window)
    pa_decode_fp8(CacheDesc.of(k_pool), out, q, k_pool, v_pool, k_scale, v_scale, block_table,
                  context_lens, max_context_len, scale, window, partition_size, workspace, err_flag,
                  stream)
    return out


def decode_append_fp8(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, max_context_len: int,
                      scale: float, key, value, slot_mapping, partition_size: int = 0, out=None, workspace=None,
                      err_flag=None, stream=None):
    """reshape_and_cache_fp8 of one token per sequence (rows in q's dtype), then decode_fp8 over
    the grown contexts, in one launch."""
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = workspace_for(k_pool, q.shape[0], q.shape[1], max_context_len, partition_size)
    pa_decode_append_fp8(CacheDesc.of(k_pool), out, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                         max_context_len, scale, key, value, slot_mapping, partition_size, workspace, err_flag, stream)
    return out


def decode_beams(q, k_pool, v_pool, block_table, context_lens, max_context_len: int, scale: float, beam_width: int,
                 k_scale=None, v_scale=None, partition_size: int = 0, out=None, workspace=None, err_flag=None,
                 stream=None):
    """decode (or decode_fp8 when the scales are given) with sequences grouped by beam_width:
    blocks that every beam of a group lists in a partition are read once for the group."""
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        n = pa_decode_beams_workspace_bytes(CacheDesc.of(k_pool), int(q.shape[0]), int(beam_width), int(q.shape[1]),
                                            max_context_len, partition_size)
        workspace = torch.empty((n + 3) // 4, dtype=torch.float32, device=q.device) if n else None
    pa_decode_beams(CacheDesc.of(k_pool), out, q, k_pool, v_pool, block_table, context_lens, max_context_len, scale,
                    beam_width, k_scale, v_scale, partition_size, workspace, err_flag, stream)
    return out


def reshape_and_cache_fp8(key, value, k_pool, v_pool, k_scale, v_scale, slot_mapping, err_flag=None,
                          stream=None):
    pa_reshape_and_cache_fp8(CacheDesc.of(k_pool), key, value, k_pool, v_pool, k_scale, v_scale,
                             slot_mapping, err_flag, stream)


def copy_blocks_fp8(k_pool, v_pool, k_scale, v_scale, pairs, err_flag=None, stream=None):
    pa_copy_blocks_fp8(CacheDesc.of(k_pool), k_pool, v_pool, k_scale, v_scale, pairs, err_flag, stream)


def reblock(src_k, src_v, src_table, dst_k, dst_v, dst_table, context_lens, max_context_len: int,
            scales=None, err_flag=None, stream=None):
    """Copy every valid row from one paged layout to another (another block size); ``scales``
    = (src_k_scale, src_v_scale, dst_k_scale, dst_v_scale) for 8-bit pools."""
    sk = scales if scales is not None else (None, None, None, None)
    pa_reblock(CacheDesc.of(src_k), src_k, src_v, src_table, CacheDesc.of(dst_k), dst_k, dst_v, dst_table,
               context_lens, max_context_len, *sk, err_flag=err_flag, stream=stream)


def multi_token_attention(q, k_pool, v_pool, block_table, context_lens, query_start, max_context_len: int,
                          max_query_len: int, scale: float, k_scale=None, v_scale=None, partition_size: int = 0,
                          out=None, workspace=None, err_flag=None, stream=None):
    """Causal attention of several new query rows per sequence (rows query_start[b] ..
    query_start[b+1]-1, already appended to the cache) over the paged cache."""
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        n = pa_multi_token_workspace_bytes(CacheDesc.of(k_pool), int(context_lens.numel()), int(q.shape[0]),
                                           int(q.shape[1]), max_context_len, max_query_len, partition_size)
        workspace = torch.empty((n + 3) // 4, dtype=torch.float32, device=q.device) if n else None
    pa_multi_token_attention(CacheDesc.of(k_pool), out, q, k_pool, v_pool, block_table, context_lens, query_start,
                             max_context_len, max_query_len, scale, k_scale, v_scale, partition_size, workspace,
                             err_flag, stream)
    return out
