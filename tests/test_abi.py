"""C ABI: libpagedkv.so loads, exports every function include/pagedkv.h declares, and its
host-only helpers (status text, partition policy, workspace size) behave. No kernels run."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_indexed_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared():
    """Every function any include/*.h declares."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            names.update(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from paged_kv_cache_indexed_amd.build import build
        build()
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings(lib):
    assert _lib.pa_status_string(0) == "PA_OK"
    assert "INVALID" in _lib.pa_status_string(1)
    assert "UNSUPPORTED" in _lib.pa_status_string(2)
    assert "LAUNCH" in _lib.pa_status_string(3)


def _desc(bs=16, hkv=32, d=128, dtype=_lib.PA_F16, nb=1000):
    return _lib.CacheDesc(nb, bs, hkv, d, dtype)


def test_partition_policy(lib):
    c = _desc()
    # short contexts with enough (sequence, kv head) pairs: one partition, whole length
    assert _lib.pa_decode_partition_size(c, 64, 32, 521, 0) == 528
    assert _lib.pa_decode_workspace_bytes(c, 64, 32, 521, 0) == 0
    # long contexts: 512-token partitions
    assert _lib.pa_decode_partition_size(_desc(bs=32), 32, 32, 32769, 0) == 512
    # the long-tail batch (256 x 32 heads, up to 1197 tokens): 256-token partitions for
    # 16-bit rows (up to 2048-token contexts; 2049 and beyond: 512), one whole partition for
    # 8-bit rows (twice the tokens per byte)
    assert _lib.pa_decode_partition_size(c, 256, 32, 1197, 0) == 256
    assert _lib.pa_decode_partition_size(c, 256, 32, 2048, 0) == 256
    assert _lib.pa_decode_partition_size(c, 256, 32, 2049, 0) == 512
    assert _lib.pa_decode_partition_size(_desc(dtype=_lib.PA_FP8_E4M3), 256, 32, 1197, 0) == 1200
    assert _lib.pa_decode_partition_size(_desc(dtype=_lib.PA_FP8_E4M3), 256, 32, 2049, 0) == 512
    # partition records (head_dim + 2 floats) and one int32 slot per sequence
    assert _lib.pa_decode_workspace_bytes(_desc(bs=32), 32, 32, 32769, 0) == 32 * 32 * 65 * 130 * 4 + 32 * 4
    # VALU path with few workgroups: partitions shrink toward ~2048 workgroups
    p = _lib.pa_decode_partition_size(_desc(hkv=8, dtype=_lib.PA_F32), 32, 64, 2049, 0)
    assert p % 16 == 0 and 32 * 8 * -(-2049 // p) >= 2048 - 256
    # ... but not below 256 tokens: config 1 (4 sequences x 8 heads, 129 tokens) keeps one
    # partition, one sequence of 4096 tokens at 32 heads gets 16
    assert _lib.pa_decode_partition_size(_desc(hkv=8, d=64, dtype=_lib.PA_F32, nb=64), 4, 8, 129, 0) == 144
    assert _lib.pa_decode_partition_size(c, 1, 32, 4096, 0) == 256
    # matrix-core path (bf16, 8 query heads per kv head): one partition for 256 pairs
    assert _lib.pa_decode_partition_size(_desc(hkv=8, dtype=_lib.PA_BF16), 32, 64, 2049, 0) == 2064
    # ... split to reach 256 workgroups, and at most 4096 tokens per partition
    assert _lib.pa_decode_partition_size(_desc(hkv=8, dtype=_lib.PA_BF16), 4, 64, 2049, 0) == 272  # 8 parts
    p = _lib.pa_decode_partition_size(_desc(hkv=8, dtype=_lib.PA_BF16), 32, 64, 32769, 0)
    assert p <= 4096 and p % 16 == 0 and -(-32769 // p) == 9
    # explicit sizes must be block multiples and fit the LDS id table
    assert _lib.pa_decode_partition_size(c, 4, 32, 100, 24) == -1
    assert _lib.pa_decode_partition_size(c, 4, 32, 100, 64) == 64
    assert _lib.pa_decode_partition_size(_desc(bs=8), 4, 32, 100, 8192) == 8192
    assert _lib.pa_decode_partition_size(_desc(bs=8), 4, 32, 100, 8200) == -1


def test_sliding_window_sizing(lib):
    # partitions cover the window plus at most block_size - 1 tokens before it
    c = _desc(bs=32)
    span = 4096 + 31
    p = _lib.pa_decode_partition_size(c, 32, 32, span, 0)
    want = 32 * 32 * -(-span // p) * 130 * 4 + 32 * 4 if -(-span // p) > 1 else 0
    assert _lib.pa_decode_sliding_window_workspace_bytes(c, 32, 32, 32769, 4096, 0) == want
    # a window at least as long as every context sizes exactly like the full decode
    for w in (32769, 40000, 2**31 - 1):
        assert (_lib.pa_decode_sliding_window_workspace_bytes(c, 32, 32, 32769, w, 0)
                == _lib.pa_decode_workspace_bytes(c, 32, 32, 32769, 0))
    # explicit partition sizes
    assert (_lib.pa_decode_sliding_window_workspace_bytes(c, 2, 4, 10000, 1000, 256)
            == 2 * 4 * -(-(1000 + 31) // 256) * 130 * 4 + 2 * 4)
    # never more than the full decode needs
    for w in (1, 7, 33, 500, 1024, 5000):
        for P in (0, 32, 128, 512):
            assert (_lib.pa_decode_sliding_window_workspace_bytes(c, 8, 32, 9000, w, P)
                    <= _lib.pa_decode_workspace_bytes(c, 8, 32, 9000, P))
    assert _lib.pa_decode_sliding_window_workspace_bytes(c, 8, 32, 9000, 0, 0) == 0
    d = c.c()
    st = lib.pa_decode_sliding_window(ctypes.byref(d), None, None, None, None, None, 4, None, 0, 32, 10,
                                      1.0, 0, 0, None, 0, None, None)
    assert st == _lib.PA_ERR_INVALID_ARGUMENT  # window 0


def test_unsupported_and_invalid_caches(lib):
    assert _lib.pa_decode_partition_size(_desc(bs=12), 4, 32, 100, 0) == -1
    assert _lib.pa_decode_partition_size(_desc(d=96), 4, 32, 100, 0) == -1
    assert _lib.pa_decode_partition_size(_desc(dtype=7), 4, 32, 100, 0) == -1
    # argument errors come back before any launch (null pointers; batch 0 is a no-op)
    d = _desc().c()
    st = lib.pa_decode(ctypes.byref(d), None, None, None, None, None, 4, None, 2, 32, 10, 1.0,
                       0, None, 0, None, None)
    assert st == _lib.PA_ERR_INVALID_ARGUMENT
    st = lib.pa_decode(ctypes.byref(d), None, None, None, None, None, 4, None, 0, 32, 10, 1.0,
                       0, None, 0, None, None)
    assert st == _lib.PA_OK
    st = lib.pa_reshape_and_cache(ctypes.byref(d), None, None, None, None, None, 0, None, None)
    assert st == _lib.PA_OK
    st = lib.pa_copy_blocks(ctypes.byref(d), None, None, None, -1, None, None)
    assert st == _lib.PA_ERR_INVALID_ARGUMENT
    bad = _desc(bs=1024).c()
    st = lib.pa_copy_blocks(ctypes.byref(bad), None, None, None, 0, None, None)
    assert st == _lib.PA_ERR_UNSUPPORTED
