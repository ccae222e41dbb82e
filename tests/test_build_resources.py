"""The compiler's per-kernel resource report of the last build: no kernel spills registers to
scratch memory (a spill in the streaming loop cost 8x once), and the decode kernels keep the
occupancy they are tuned for. CPU only; skipped when nothing has been built here."""

import csv
import os

import pytest

from paged_kv_cache_indexed_amd.build import RESOURCES_PATH

pytestmark = pytest.mark.skipif(not os.path.exists(RESOURCES_PATH), reason="no build in this tree")


def _rows():
    with open(RESOURCES_PATH) as f:
        return list(csv.DictReader(f, delimiter="\t"))


def test_every_kernel_reported():
    names = " ".join(r["kernel"] for r in _rows())
    for k in ("decode_valu_kernel", "decode_valu_heads_kernel", "decode_mfma_kernel", "prefill_kernel",
              "reduce_kernel", "reduce_multi_kernel", "reshape_and_cache_kernel", "copy_blocks_kernel"):
        assert k in names, k


def test_no_kernel_spills():
    spills = [(r["kernel"], r["scratch_bytes_per_lane"]) for r in _rows() if int(r["scratch_bytes_per_lane"]) != 0]
    assert not spills, spills[:10]


def test_decode_occupancy():
    for r in _rows():
        occ = int(r["occupancy_waves_per_simd"])
        # the 8-token-block decode with per-lane addresses over 16-bit rows of 128 dims holds a
        # 64-bit address per lane and row; it asks for one wave per SIMD rather than spill
        small16 = "Li128E" in r["kernel"] and "ELb0ELb0ELi1EE" in r["kernel"] and "FP8" not in r["kernel"]
        if "decode_mfma_kernel" in r["kernel"] or "prefill_kernel" in r["kernel"]:
            assert occ >= (1 if small16 else 2), (r["kernel"], occ)
