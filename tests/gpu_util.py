"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from paged_kv_cache_indexed_amd import ops

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}


def note(msg: str) -> None:
    """Name the case on stdout before each GPU step, so a failure is attributable."""
    print(f"[gpu-case] {msg}", flush=True)


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    return torch.device("cuda", 0)


def gpu_decode(w, dev, lens=None, partition_size=0, tensors=None, err_flag=None):
    """Run pa_decode on workload ``w``; returns (float64 numpy output, device output)."""
    t = tensors if tensors is not None else w.to_device(dev)
    lens_t = t["context_lens"] if lens is None else torch.as_tensor(lens, dtype=torch.int32, device=dev)
    max_len = int(lens_t.max().item())
    out = ops.decode(t["q"], t["k_pool"], t["v_pool"], t["block_table"], lens_t, max_len, w.scale,
                     partition_size=partition_size, err_flag=err_flag)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), out


def oracle_decode(w, lens=None, k_pool=None, v_pool=None, table=None):
    return oracle.paged_decode(w.q, w.k_pool if k_pool is None else k_pool,
                               w.v_pool if v_pool is None else v_pool,
                               w.block_table if table is None else table,
                               w.context_lens if lens is None else lens, w.scale)


def max_err(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


# Every comparison of this process: (what, dtype, raw max-abs error, error beyond the output
# rounding); the session summary lists them (tests/conftest.py).
RESULTS: list = []

# Half an ulp relative to |o| of the output type: the one rounding of the fp32 result.
HALF_ULP = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def assert_close(got, ref, dtype: str, what: str) -> float:
    """Elementwise |got - ref| <= TOL + |ref| * HALF_ULP: the max-abs tolerance bounds the fp32
    result, and its final rounding to the output type adds at most half an ulp of |o|."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    err = float(diff.max()) if diff.size else 0.0
    excess = float(np.max(diff - np.abs(ref) * HALF_ULP[dtype])) if diff.size else 0.0
    print(f"[gpu-result] {what}: max abs err {err:.3e}, beyond output rounding {excess:.3e} "
          f"(tol {TOL[dtype]:.0e})", flush=True)
    RESULTS.append((what, dtype, err, excess))
    assert excess <= TOL[dtype], f"{what}: error beyond output rounding {excess:.3e} > {TOL[dtype]}"
    return err


def flush_print():
    sys.stdout.flush()
