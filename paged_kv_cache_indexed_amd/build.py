"""Build libpagedkv.so for gfx950 with hipcc (cross-compiles without a GPU).

    python -m paged_kv_cache_indexed_amd.build          # writes paged_kv_cache_indexed_amd/libpagedkv.so
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpagedkv.so")
# per-kernel registers, scratch, LDS and occupancy of the last build (from the compiler's
# resource-usage remarks)
RESOURCES_PATH = os.path.join(BUILD_DIR, "kernel_resources.tsv")
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of the generated code: every HIP compile disables the
# target feature that lets the backend form them.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


_REMARK = re.compile(r"remark: .*?Function Name: (\S+)|remark: .*?(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\d+)")


def _resources(stderr: str):
    """(kernel, vgprs, agprs, scratch bytes per lane, occupancy, LDS bytes) from the remarks."""
    rows, cur = [], None
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        if m.group(1):
            cur = {"name": m.group(1)}
            rows.append(cur)
        elif cur is not None:
            cur[m.group(2).split()[0]] = int(m.group(3))
    return [(r["name"], r.get("VGPRs", -1), r.get("AGPRs", -1), r.get("ScratchSize", -1), r.get("Occupancy", -1),
             r.get("LDS", -1)) for r in rows]


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every csrc/*.hip for gfx950 and link libpagedkv.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        done = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [o for o, _ in done]
    with open(RESOURCES_PATH, "w") as f:
        f.write("kernel\tvgprs\tagprs\tscratch_bytes_per_lane\toccupancy_waves_per_simd\tlds_bytes\n")
        for _, rows in done:
            for row in rows:
                f.write("\t".join(str(x) for x in row) + "\n")
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
