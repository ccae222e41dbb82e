"""Seeded synthetic inputs for paged-KV decode.

This package only draws random numbers and lays them out: contiguous per-sequence K/V
contents, a shuffled physical block pool, block tables, lengths, append slots and
copy-on-write pairs. It contains none of the attention arithmetic, so both the CPU
oracle's tests and the HIP path's tests may use it without sharing any computation.
"""

from .paged import (  # noqa: F401
    DTYPE_BYTES,
    PagedWorkload,
    build_paged,
    config_workload,
    cast_like,
    lognormal_lengths,
    DevicePagedWorkload,
    config3_device_family,
    config3_lengths,
    device_paged,
    paged_contents,
)
