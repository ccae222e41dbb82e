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
        # the 8-token-block kernels with per-lane addresses (last template argument 1) over
        # rows of 128 dims hold a 64-bit address per lane and row; with 16-bit rows, or in the
        # multi-token and beam-group modes, they ask for one wave per SIMD rather than spill
        k = r["kernel"]
        per_lane = "Li128E" in k and k.endswith("ELi1EEEvNS_10DecodeArgsE")
        small = per_lane and ("FP8" not in k or "ELb1ELb1ELb0ELi1EE" in k or "ELb1ELb0ELb1ELi1EE" in k)
        if "decode_mfma_kernel" in k or "prefill_kernel" in k:
            assert occ >= (1 if small else 2), (k, occ)
