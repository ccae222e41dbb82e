"""CPU oracle for paged-KV decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. It is never on the product path, and it shares no code with the
HIP library: it is written from the pages' description of what PagedAttention computes.
``oracle.fp8_cache`` covers blocks stored as 8-bit floats with a scale per row.
"""

from .paged_attention import (  # noqa: F401
    OracleInputError,
    allocated_kv_bytes,
    attention_one_query,
    blocks_needed,
    compact_blocks,
    copy_blocks,
    gather_range,
    gather_sequence,
    kv_cache_bytes,
    layer_pools,
    paged_attention_multi,
    paged_decode,
    paged_decode_heads,
    paged_decode_window,
    window_start,
    reblock,
    reshape_and_cache,
)

from . import fp8_cache  # noqa: F401,E402
