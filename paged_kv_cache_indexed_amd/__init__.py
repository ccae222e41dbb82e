"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute lives in libpagedkv.so (hand-written HIP kernels behind the C ABI of
include/pagedkv.h). This package holds its thin ctypes binding (``_lib``), the build script
(``build``), a convenience layer that allocates outputs and workspaces with torch
(``ops``) and the host-side block manager (``block_manager``).
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    CacheDesc,
    PagedKVError,
    pa_copy_blocks,
    pa_copy_blocks_fp8,
    pa_decode,
    pa_decode_append,
    pa_decode_append_fp8,
    pa_decode_beams,
    pa_decode_beams_partition_size,
    pa_decode_beams_workspace_bytes,
    pa_decode_fp8,
    pa_decode_partition_size,
    pa_decode_sliding_window,
    pa_decode_sliding_window_workspace_bytes,
    pa_decode_workspace_bytes,
    pa_multi_token_attention,
    pa_multi_token_workspace_bytes,
    pa_reblock,
    pa_reshape_and_cache,
    pa_reshape_and_cache_fp8,
    pa_status_string,
)
