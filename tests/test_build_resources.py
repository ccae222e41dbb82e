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


def test_lds_path_occupancy():
    """The LDS-path decode keeps four waves per SIMD, and its work-groups fit the LDS that
    occupancy needs: two 8-wave or four 4-wave work-groups per compute unit (160 KB)."""
    rows = [r for r in _rows() if "decode_mfma_lds_kernel" in r["kernel"]]
    assert rows
    for r in rows:
        nw = 8 if "ELi8EEEvNS_10DecodeArgsE" in r["kernel"] else 4
        assert int(r["occupancy_waves_per_simd"]) == 4, r["kernel"]
        assert int(r["lds_bytes"]) * (16 // nw) <= 160 * 1024, (r["kernel"], r["lds_bytes"])


def test_valu_occupancy():
    """The VALU stream kernels at one query head per kv head keep the waves per SIMD they were
    measured at: with 16-bit pools at head_dim 128, 8 for fp16 (64 registers) and 7 for bf16;
    with 8-bit pools, 7 (a lane's 16 codes per load, 72 registers)."""
    import re

    pat = re.compile(r"decode_valu_kernelINS_(3F16|4BF16)E(NS_3FP8E|S2_)Li(\d+)ELi1ELi(\d)ELi4E")
    seen = set()
    for r in _rows():
        m = pat.search(r["kernel"])
        if not m:
            continue
        q, kv, d, unroll = m.group(1), m.group(2), int(m.group(3)), int(m.group(4))
        occ = int(r["occupancy_waves_per_simd"])
        if kv == "NS_3FP8E":
            seen.add("fp8")
            assert occ >= 7, (r["kernel"], occ)
        elif d == 128 and unroll == 2:
            seen.add(q)
            assert occ >= (8 if q == "3F16" else 7), (r["kernel"], occ)
    assert seen == {"fp8", "3F16", "4BF16"}, seen


def _device_asm(src: str) -> str:
    """The device assembly of one source file of the library (compiled here, for gfx950)."""
    import shutil
    import subprocess
    import tempfile

    from paged_kv_cache_indexed_amd import build

    if shutil.which(build._hipcc()) is None and not os.path.exists(build._hipcc()):
        pytest.skip("no hipcc")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [build._hipcc(), *[f for f in build.HIP_FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
               os.path.join(build.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return f.read()


def _function(asm: str, name_part: str) -> str:
    start = next(i for i, line in enumerate(asm.splitlines())
                 if line.split(";")[0].strip().endswith(":") and name_part in line and not line.startswith((".", "\t")))
    body = []
    for line in asm.splitlines()[start + 1:]:
        body.append(line)
        if "s_endpgm" in line:
            break
    return "\n".join(body)


def test_measurement_kernels_load_full_width():
    """The read-rate kernels must move the bytes they claim to: every buffer load of the
    gather and every load of the streaming loop is 16 bytes per lane. (If some dwords of a
    load feed nothing, the compiler narrows it, and the measured rate is of another access.)"""
    import re

    asm = _device_asm("pa_measure.hip")
    gather = _function(asm, "gather_read_kernel")
    loads = re.findall(r"buffer_load_dword\w*", gather)
    assert loads and set(loads) == {"buffer_load_dwordx4"}, sorted(set(loads))
    stream = _function(asm, "stream_read_kernel")
    assert len(re.findall(r"global_load_dwordx4", stream)) >= 8
    assert not re.findall(r"global_load_dword(?:x2|x3)?\s", stream)
