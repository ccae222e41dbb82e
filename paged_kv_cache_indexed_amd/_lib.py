"""ctypes binding of libpagedkv (include/pagedkv.h): argument marshalling only.

Every function has the name of the C entry point it calls. Tensors are torch tensors on the
GPU; only their data pointers, shapes and the current HIP stream cross the boundary. All
computation happens in the library's HIP kernels. If libpagedkv.so is missing the first
call raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build. PAGEDKV_LIB selects another build of the same library (a tuning
# variant); bench.py refuses it unless asked for one, and every record names the library
# it loaded with its hash (library_identity()).
DEFAULT_LIB_PATH = os.path.join(_PKG, "libpagedkv.so")
LIB_PATH = os.environ.get("PAGEDKV_LIB") or DEFAULT_LIB_PATH

PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_UNSUPPORTED, PA_ERR_LAUNCH, PA_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
PA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/pagedkv.h
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_FLAG_BAD_BLOCK_ID = 1
PA_FLAG_BAD_LENGTH = 2
PA_FLAG_EMPTY_CONTEXT = 4
PA_FLAG_BAD_SLOT = 8
PA_FLAG_BAD_COPY_PAIR = 16

EXPORTED = ("pa_reshape_and_cache", "pa_copy_blocks", "pa_decode_partition_size",
            "pa_decode_workspace_bytes", "pa_decode", "pa_decode_sliding_window",
            "pa_decode_sliding_window_workspace_bytes", "pa_reshape_and_cache_fp8",
            "pa_copy_blocks_fp8", "pa_decode_fp8", "pa_reblock", "pa_multi_token_attention",
            "pa_multi_token_workspace_bytes", "pa_decode_append", "pa_decode_append_fp8",
            "pa_decode_beams", "pa_decode_beams_partition_size", "pa_decode_beams_workspace_bytes",
            "pa_status_string", "pa_measure_stream_read", "pa_measure_gather_read", "pa_decode_append_noalloc")

# 8-bit float pools are uint8 (or float8_e4m3fn) tensors of OCP E4M3 codes.
_DTYPE_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
               torch.uint8: PA_FP8_E4M3, torch.float8_e4m3fn: PA_FP8_E4M3}


class pa_cache_desc_t(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("block_stride", ctypes.c_int64)]


@dataclass(frozen=True)
class CacheDesc:
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    dtype: int
    block_stride: int = 0  # bytes between consecutive blocks; 0 = dense

    @staticmethod
    def of(k_pool: torch.Tensor) -> "CacheDesc":
        """Describe a [num_blocks][kv_heads][block_size][head_dim] pool tensor. Blocks must be
        dense inside; the distance between blocks (dim 0's stride) may be larger, as for one
        layer's K or V in a [blocks][2][layers][heads][block_size][head_dim] allocation."""
        nb, hkv, bs, d = k_pool.shape
        _check_pool_layout(k_pool)
        dense = hkv * bs * d
        stride = int(k_pool.stride(0))
        return CacheDesc(int(nb), int(bs), int(hkv), int(d), _DTYPE_CODE[k_pool.dtype],
                         0 if stride == dense else stride * k_pool.element_size())

    def c(self) -> pa_cache_desc_t:
        return pa_cache_desc_t(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim,
                               self.dtype, self.block_stride)


class PagedKVError(RuntimeError):
    pass


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpagedkv.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise PagedKVError(f"{path} is missing: build it with python -m paged_kv_cache_indexed_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(pa_cache_desc_t)
    lib.pa_reshape_and_cache.argtypes = [D, P, P, P, P, P, I32, P, P]
    lib.pa_reshape_and_cache.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [D, P, P, P, I32, P, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_decode_partition_size.argtypes = [D, I32, I32, I32, I32]
    lib.pa_decode_partition_size.restype = I32
    lib.pa_decode_workspace_bytes.argtypes = [D, I32, I32, I32, I32]
    lib.pa_decode_workspace_bytes.restype = SZ
    lib.pa_decode.argtypes = [D, P, P, P, P, P, I32, P, I32, I32, I32, F, I32, P, SZ, P, P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_sliding_window.argtypes = [D, P, P, P, P, P, I32, P, I32, I32, I32, F, I32, I32, P, SZ, P, P]
    lib.pa_decode_sliding_window.restype = ctypes.c_int
    lib.pa_decode_sliding_window_workspace_bytes.argtypes = [D, I32, I32, I32, I32, I32]
    lib.pa_decode_sliding_window_workspace_bytes.restype = SZ
    lib.pa_reshape_and_cache_fp8.argtypes = [D, I32, P, P, P, P, P, P, P, I32, P, P]
    lib.pa_reshape_and_cache_fp8.restype = ctypes.c_int
    lib.pa_copy_blocks_fp8.argtypes = [D, P, P, P, P, P, I32, P, P]
    lib.pa_copy_blocks_fp8.restype = ctypes.c_int
    lib.pa_decode_fp8.argtypes = [D, I32, P, P, P, P, P, P, P, I32, P, I32, I32, I32, F, I32, I32, P, SZ, P, P]
    lib.pa_decode_fp8.restype = ctypes.c_int
    lib.pa_reblock.argtypes = [D, P, P, P, P, P, I32, D, P, P, P, P, P, I32, P, I32, I32, P, P]
    lib.pa_reblock.restype = ctypes.c_int
    lib.pa_multi_token_attention.argtypes = [D, I32, P, P, P, P, P, P, P, I32, P, P, I32, I32, I32, I32, I32, F,
                                             I32, P, SZ, P, P]
    lib.pa_multi_token_attention.restype = ctypes.c_int
    lib.pa_multi_token_workspace_bytes.argtypes = [D, I32, I32, I32, I32, I32, I32]
    lib.pa_multi_token_workspace_bytes.restype = SZ
    lib.pa_decode_append.argtypes = [D, P, P, P, P, P, I32, P, I32, I32, I32, F, P, P, P, I32, P, SZ, P, P]
    lib.pa_decode_append.restype = ctypes.c_int
    lib.pa_decode_append_fp8.argtypes = [D, I32, P, P, P, P, P, P, P, I32, P, I32, I32, I32, F, P, P, P, I32, P, SZ,
                                         P, P]
    lib.pa_decode_append_fp8.restype = ctypes.c_int
    lib.pa_decode_beams.argtypes = [D, I32, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, F, I32, P, SZ, P, P]
    lib.pa_decode_beams.restype = ctypes.c_int
    lib.pa_decode_beams_partition_size.argtypes = [D, I32, I32, I32, I32, I32]
    lib.pa_decode_beams_partition_size.restype = I32
    lib.pa_decode_beams_workspace_bytes.argtypes = [D, I32, I32, I32, I32, I32]
    lib.pa_decode_beams_workspace_bytes.restype = SZ
    lib.pa_decode_append_noalloc.argtypes = [D, P, P, P, P, P, I32, P, I32, I32, I32, F, P, P, P, I32, P, P]
    lib.pa_decode_append_noalloc.restype = ctypes.c_int
    lib.pa_measure_stream_read.argtypes = [P, SZ, P, I32, P]
    lib.pa_measure_stream_read.restype = ctypes.c_int
    lib.pa_measure_gather_read.argtypes = [D, P, P, P, I32, P, I32, I32, P, P]
    lib.pa_measure_gather_read.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library_identity(path: str = LIB_PATH) -> dict:
    """Path and sha256 (first 16 hex digits) of the library file, and whether it is the
    in-tree build."""
    import hashlib

    h = hashlib.sha256()
    with open(path, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 20), b""):
            h.update(chunk)
    return {"path": os.path.relpath(path, os.path.dirname(_PKG)) if path.startswith(os.path.dirname(_PKG))
            else path, "sha256_16": h.hexdigest()[:16],
            "in_tree": os.path.abspath(path) == os.path.abspath(DEFAULT_LIB_PATH)}


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise PagedKVError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise PagedKVError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check_pool_layout(t) -> None:
    nb, hkv, bs, d = t.shape
    if t.stride(3) != 1 or t.stride(2) != d or t.stride(1) != bs * d or (nb > 1 and t.stride(0) < hkv * bs * d):
        raise PagedKVError("pool blocks must be dense [kv_heads][block_size][head_dim] slabs")


def _pool_ptr(t, like=None):
    """Pointer of a pool tensor whose blocks may be strided (dim 0) but are dense inside."""
    if not t.is_cuda:
        raise PagedKVError("tensor must live on the GPU")
    _check_pool_layout(t)
    if like is not None and t.stride() != like.stride():
        raise PagedKVError("k_pool and v_pool must have the same layout")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int) -> None:
    if status != PA_OK:
        raise PagedKVError(pa_status_string(status))


def pa_status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def pa_reshape_and_cache(cache: CacheDesc, key, value, k_pool, v_pool, slot_mapping,
                         err_flag=None, stream=None) -> None:
    n = int(slot_mapping.numel())
    desc = cache.c()
    _check(load().pa_reshape_and_cache(ctypes.byref(desc), _ptr(key), _ptr(value), _pool_ptr(k_pool),
                                       _pool_ptr(v_pool, k_pool), _ptr(slot_mapping), n, _ptr(err_flag),
                                       _stream(stream)))


def pa_copy_blocks(cache: CacheDesc, k_pool, v_pool, pairs, err_flag=None, stream=None) -> None:
    n = int(pairs.shape[0]) if pairs is not None else 0
    desc = cache.c()
    _check(load().pa_copy_blocks(ctypes.byref(desc), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool),
                                 _ptr(pairs) if n else None, n, _ptr(err_flag), _stream(stream)))


def pa_decode_partition_size(cache: CacheDesc, batch: int, num_q_heads: int, max_context_len: int,
                             requested: int = 0) -> int:
    desc = cache.c()
    return int(load().pa_decode_partition_size(ctypes.byref(desc), batch, num_q_heads,
                                               max_context_len, requested))


def pa_decode_workspace_bytes(cache: CacheDesc, batch: int, num_q_heads: int, max_context_len: int,
                              partition_size: int = 0) -> int:
    desc = cache.c()
    return int(load().pa_decode_workspace_bytes(ctypes.byref(desc), batch, num_q_heads,
                                                max_context_len, partition_size))


def pa_decode_sliding_window_workspace_bytes(cache: CacheDesc, batch: int, num_q_heads: int,
                                             max_context_len: int, window: int,
                                             partition_size: int = 0) -> int:
    desc = cache.c()
    return int(load().pa_decode_sliding_window_workspace_bytes(
        ctypes.byref(desc), batch, num_q_heads, max_context_len, window, partition_size))


def pa_decode(cache: CacheDesc, out, q, k_pool, v_pool, block_table, context_lens,
              max_context_len: int, scale: float, partition_size: int = 0, workspace=None,
              err_flag=None, stream=None) -> None:
    batch, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache.c()
    _check(load().pa_decode(ctypes.byref(desc), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool),
                            _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens),
                            batch, num_q_heads, int(max_context_len), float(scale),
                            int(partition_size), _ptr(workspace), ws_bytes, _ptr(err_flag),
                            _stream(stream)))


def pa_decode_sliding_window(cache: CacheDesc, out, q, k_pool, v_pool, block_table, context_lens,
                             max_context_len: int, scale: float, window: int, partition_size: int = 0,
                             workspace=None, err_flag=None, stream=None) -> None:
    batch, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache.c()
    _check(load().pa_decode_sliding_window(
        ctypes.byref(desc), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool), _ptr(block_table),
        int(block_table.shape[1]), _ptr(context_lens), batch, num_q_heads, int(max_context_len),
        float(scale), int(window), int(partition_size), _ptr(workspace), ws_bytes, _ptr(err_flag),
        _stream(stream)))


def dtype_code(t: torch.Tensor) -> int:
    return _DTYPE_CODE[t.dtype]


def pa_reshape_and_cache_fp8(cache: CacheDesc, key, value, k_pool, v_pool, k_scale, v_scale, slot_mapping,
                             err_flag=None, stream=None) -> None:
    n = int(slot_mapping.numel())
    desc = cache.c()
    _check(load().pa_reshape_and_cache_fp8(ctypes.byref(desc), dtype_code(key), _ptr(key), _ptr(value),
                                           _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool), _ptr(k_scale), _ptr(v_scale),
                                           _ptr(slot_mapping), n, _ptr(err_flag), _stream(stream)))


def pa_copy_blocks_fp8(cache: CacheDesc, k_pool, v_pool, k_scale, v_scale, pairs, err_flag=None,
                       stream=None) -> None:
    n = int(pairs.shape[0]) if pairs is not None else 0
    desc = cache.c()
    _check(load().pa_copy_blocks_fp8(ctypes.byref(desc), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(pairs) if n else None, n, _ptr(err_flag),
                                     _stream(stream)))


def pa_decode_fp8(cache: CacheDesc, out, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                  max_context_len: int, scale: float, window: int = 0, partition_size: int = 0,
                  workspace=None, err_flag=None, stream=None) -> None:
    batch, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache.c()
    _check(load().pa_decode_fp8(
        ctypes.byref(desc), dtype_code(q), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), batch, num_q_heads,
        int(max_context_len), float(scale), int(window), int(partition_size), _ptr(workspace), ws_bytes,
        _ptr(err_flag), _stream(stream)))


def pa_reblock(src: CacheDesc, src_k, src_v, src_table, dst: CacheDesc, dst_k, dst_v, dst_table, context_lens,
               max_context_len: int, src_k_scale=None, src_v_scale=None, dst_k_scale=None, dst_v_scale=None,
               err_flag=None, stream=None) -> None:
    sd, dd = src.c(), dst.c()
    _check(load().pa_reblock(
        ctypes.byref(sd), _pool_ptr(src_k), _pool_ptr(src_v, src_k), _ptr(src_k_scale), _ptr(src_v_scale),
        _ptr(src_table), int(src_table.shape[1]), ctypes.byref(dd), _pool_ptr(dst_k), _pool_ptr(dst_v, dst_k),
        _ptr(dst_k_scale), _ptr(dst_v_scale), _ptr(dst_table), int(dst_table.shape[1]), _ptr(context_lens),
        int(context_lens.numel()), int(max_context_len), _ptr(err_flag), _stream(stream)))


def pa_multi_token_workspace_bytes(cache: CacheDesc, batch: int, num_q_tokens: int, num_q_heads: int,
                                   max_context_len: int, max_query_len: int, partition_size: int = 0) -> int:
    desc = cache.c()
    return int(load().pa_multi_token_workspace_bytes(ctypes.byref(desc), batch, num_q_tokens, num_q_heads,
                                                      max_context_len, max_query_len, partition_size))


def pa_multi_token_attention(cache: CacheDesc, out, q, k_pool, v_pool, block_table, context_lens, query_start,
                             max_context_len: int, max_query_len: int, scale: float, k_scale=None, v_scale=None,
                             partition_size: int = 0, workspace=None, err_flag=None, stream=None) -> None:
    num_q_tokens, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache.c()
    _check(load().pa_multi_token_attention(
        ctypes.byref(desc), dtype_code(q), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens),
        _ptr(query_start), int(context_lens.numel()), num_q_tokens, num_q_heads, int(max_context_len),
        int(max_query_len), float(scale), int(partition_size), _ptr(workspace), ws_bytes, _ptr(err_flag),
        _stream(stream)))


def pa_decode_append_fp8(cache: CacheDesc, out, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                         max_context_len: int, scale: float, key, value, slot_mapping, partition_size: int = 0,
                         workspace=None, err_flag=None, stream=None) -> None:
    batch, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache.c()
    _check(load().pa_decode_append_fp8(
        ctypes.byref(desc), dtype_code(q), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), batch,
        num_q_heads, int(max_context_len), float(scale), _ptr(key), _ptr(value), _ptr(slot_mapping),
        int(partition_size), _ptr(workspace), ws_bytes, _ptr(err_flag), _stream(stream)))


def pa_decode_beams_partition_size(cache: CacheDesc, batch: int, beam_width: int, num_q_heads: int,
                                   max_context_len: int, requested: int = 0) -> int:
    desc = cache.c()
    return int(load().pa_decode_beams_partition_size(ctypes.byref(desc), batch, beam_width, num_q_heads,
                                                      max_context_len, requested))


def pa_decode_beams_workspace_bytes(cache: CacheDesc, batch: int, beam_width: int, num_q_heads: int,
                                    max_context_len: int, partition_size: int = 0) -> int:
    desc = cache.c()
    return int(load().pa_decode_beams_workspace_bytes(ctypes.byref(desc), batch, beam_width, num_q_heads,
                                                       max_context_len, partition_size))


def pa_decode_beams(cache: CacheDesc, out, q, k_pool, v_pool, block_table, context_lens, max_context_len: int,
                    scale: float, beam_width: int, k_scale=None, v_scale=None, partition_size: int = 0,
                    workspace=None, err_flag=None, stream=None) -> None:
    batch, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache.c()
    _check(load().pa_decode_beams(
        ctypes.byref(desc), dtype_code(q), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), batch,
        int(beam_width), num_q_heads, int(max_context_len), float(scale), int(partition_size), _ptr(workspace),
        ws_bytes, _ptr(err_flag), _stream(stream)))


def pa_decode_append(cache: CacheDesc, out, q, k_pool, v_pool, block_table, context_lens, max_context_len: int,
                     scale: float, key, value, slot_mapping, partition_size: int = 0, workspace=None, err_flag=None,
                     stream=None) -> None:
    batch, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache.c()
    _check(load().pa_decode_append(
        ctypes.byref(desc), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool), _ptr(block_table),
        int(block_table.shape[1]), _ptr(context_lens), batch, num_q_heads, int(max_context_len), float(scale),
        _ptr(key), _ptr(value), _ptr(slot_mapping), int(partition_size), _ptr(workspace), ws_bytes, _ptr(err_flag),
        _stream(stream)))


def pa_measure_stream_read(buf, sink, num_workgroups: int, stream=None) -> None:
    """One streaming read of the whole of ``buf`` (include/pagedkv_measure.h); ``sink`` holds
    at least ``num_workgroups`` float32."""
    if sink.numel() < num_workgroups or sink.dtype != torch.float32:
        raise PagedKVError("sink must hold num_workgroups float32")
    _check(load().pa_measure_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                         int(num_workgroups), _stream(stream)))


def pa_measure_gather_read(cache: CacheDesc, k_pool, v_pool, block_table, context_lens, max_context_len: int,
                           sink, stream=None) -> None:
    """The split decode's K/V reads of a paged cache without its arithmetic
    (include/pagedkv_measure.h); ``sink`` holds at least batch x num_kv_heads float32."""
    batch = int(context_lens.shape[0])
    if sink.numel() < batch * cache.num_kv_heads or sink.dtype != torch.float32:
        raise PagedKVError("sink must hold batch x num_kv_heads float32")
    desc = cache.c()
    _check(load().pa_measure_gather_read(ctypes.byref(desc), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool),
                                         _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), batch,
                                         int(max_context_len), _ptr(sink), _stream(stream)))


def pa_decode_append_noalloc(cache: CacheDesc, out, q, k_pool, v_pool, block_table, context_lens,
                             max_context_len: int, scale: float, key, value, slot_mapping, partition_size: int = 0,
                             err_flag=None, stream=None) -> None:
    """pa_decode_append with the library's static scratch in place of a workspace."""
    batch, num_q_heads = int(q.shape[0]), int(q.shape[1])
    desc = cache.c()
    _check(load().pa_decode_append_noalloc(
        ctypes.byref(desc), _ptr(out), _ptr(q), _pool_ptr(k_pool), _pool_ptr(v_pool, k_pool), _ptr(block_table),
        int(block_table.shape[1]), _ptr(context_lens), batch, num_q_heads, int(max_context_len), float(scale),
        _ptr(key), _ptr(value), _ptr(slot_mapping), int(partition_size), _ptr(err_flag), _stream(stream)))
