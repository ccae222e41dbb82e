"""Paged-KV decode benchmark on one MI355X.

One step = the whole hot path over one batch: copy-on-write of shared blocks (when the
workload has any), append of one new token per sequence through its slot, then decode over
the grown context. Append and decode are fused (pa_decode_append, pa_decode_append_fp8)
without a window, else pa_reshape_and_cache[_fp8] then the decode. Inputs are seeded synthetic tensors
already resident in HBM. Pools are replicated R times and step i uses replica i % R, so the
bytes touched between two reads of a replica exceed the 256 MB Infinity Cache and the
per-XCD L2 (a cold-cache measurement).

Prints one JSON line: effective KV GB/s of the whole step (algorithmic K+V bytes of the
decode, 2 x kv_heads x head_dim x dtype_bytes x sum(context_len), over the step time),
plus the decode kernel's roofline figure and the CPU oracle's rate. The K timed steps run
back to back with nothing else on the stream (--graph replays one captured HIP graph per
replica instead). The decode kernel's average launch duration comes from a second pass: K
back-to-back launches of it alone (same inputs, same replica rotation) between one pair of
HIP events on its stream. An event pair around every launch would add 2-5 us to each measured launch, and one
inside every step about 7 us to the step.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 3] [--median 87] [--block-size 16]

The default workload is the long-tail block-size sweep's median-87, 16-token-block case
(256 sequences, 32 heads, head_dim 128, fp16). With it the line also carries `sweep`: the
fused step at medians 87 and 23 and block sizes 8, 16, 32 and 64, each with its decode
launch time, GB/s, share of the 8 TB/s roofline and the time of the same cache's reads
alone (pa_measure_gather_read: the split decode's loads through the table, no arithmetic);
and `config1`: the tiny fp32 workload's step, decode launch and roofline share, with its own
oracle baseline. `roofline.ceiling` is the streaming-read rate this GPU reaches with the
library's read kernel (pa_measure_stream_read over 4 GiB), `roofline.gather_ceiling` the
rate of the decode's own reads of this cache alone (16-bit pools without a window or beam
groups), and `*_per_launch_events` give the median, p10 and p90 of launches timed one by
one.

With --window W the decode attends to the last W tokens of each sequence only
(pa_decode_sliding_window) and the algorithmic bytes count min(context_len, W) tokens.
With --kv fp8 the pools hold 8-bit floats (OCP E4M3) with a float32 scale per (token, kv
head) row, filled by the library's own quantising append; the step uses the *_fp8 entry
points and the algorithmic bytes are 2 x kv_heads x (head_dim + 4) per attended token.
With --beams W the decode is pa_decode_beams with groups of W consecutive sequences (the
append is a separate pa_reshape_and_cache[_fp8] call); config 5's groups of 4 beams share a
30720-token prefix, and its step uses pa_decode_beams with W = 4 unless --beams 0 is given. With --queries N the step appends N tokens per sequence and runs
pa_multi_token_attention over them (metric: query tokens/s).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_hbm_traffic.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "gqa_mfma_busy.txt")


# Sources each decode kernel is built from: a recorded counter figure stays valid while the
# sources of the kernel that produced it are unchanged.
_COMMON_SOURCES = ("pa_device.h", "pa_kernels.h", "pa_decode_common.h", "pa_api.hip")
_PATH_SOURCES = {"valu": ("pa_decode_valu.h", "pa_decode.hip", "pa_decode_fp8.hip"),
                 "mfma": ("pa_mfma_kernel.h", "pa_mfma_lds.h", "pa_decode_mfma.hip", "pa_decode_mfma_b8.hip"),
                 "multi": ("pa_mfma_kernel.h", "pa_multi_token.hip", "pa_multi_token_b8.hip"),
                 "beams": ("pa_mfma_kernel.h", "pa_decode_beams.hip", "pa_decode_beams_b8.hip")}


def decode_path(dtype: str, head_dim: int, group: int, block_size: int) -> str:
    """Which decode kernel the library launches (its dispatch rule, restated for the record):
    the matrix cores for 4, 8 or 16 query heads per kv head over fp16/bf16/8-bit pools with
    blocks of 16+ tokens, or of 8 tokens up to head_dim 128 (16 heads only up to head_dim
    128), else the VALU kernel."""
    ok = dtype in ("f16", "bf16", "fp8") and group in (4, 8, 16) and (
        block_size >= 16 or (block_size == 8 and head_dim <= 128))
    return "mfma" if ok and not (group == 16 and head_dim > 128) else "valu"


def kernel_source_hash(path: str = "valu") -> str:
    """Hash of the sources of one decode kernel path and the ABI header."""
    import hashlib

    csrc = os.path.join(ROOT, "paged_kv_cache_indexed_amd", "csrc")
    files = [os.path.join(csrc, f) for f in _COMMON_SOURCES + _PATH_SOURCES[path]]
    files.append(os.path.join(ROOT, "include", "pagedkv.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, path: str):
    """HBM bytes per decode launch measured with rocprofv3 for this workload, if the table in
    profiles/ was taken from the current sources of its kernel; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    cur = kernel_source_hash(path)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 5 and cells[0] == workload and cells[1] == cur:
                try:
                    return int(cells[4])
                except ValueError:
                    return None
    return None


def recorded_mfma_busy(workload: str, path: str):
    """Matrix-core busy % (rocprofv3 MfmaUtil) of the attention kernel for this workload, if
    the table in profiles/ was taken from the current sources of its kernel; else None."""
    if not os.path.exists(MFMA_FILE):
        return None
    cur = kernel_source_hash(path)
    with open(MFMA_FILE) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 8 and cells[0] == workload and cells[1] == cur:
                try:
                    return float(cells[7])
                except ValueError:
                    return None
    return None


def _workload(cfg: int, block_size: int | None, median: float | None, contiguous: bool = False):
    from workloads import config_workload

    return config_workload(cfg, seed=0, block_size=block_size, median=median, contiguous=contiguous)


def padding_waste_pct(lens, block_size: int) -> float:
    """Share of the allocated slots that hold no token: 1 - sum(L) / (bs * sum(ceil(L / bs)))."""
    lens = np.asarray(lens, np.int64)
    alloc = int((-(-lens // block_size)).sum()) * block_size
    return 100.0 * (1.0 - float(lens.sum()) / alloc) if alloc else 0.0


def _describe(w) -> dict:
    L = w.lens_after_append
    return {"workload": w.name, "dtype": w.dtype, "batch": w.batch,
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "num_blocks": w.num_blocks,
            "context_len_min": int(L.min()), "context_len_max": int(L.max()),
            "context_len_sum": int(L.sum()), "padding_waste_pct": round(padding_waste_pct(L, w.block_size), 2),
            "step": "append 1 token/seq + decode"}


def _cpu_baseline(w, budget_s: float, window: int = 0) -> dict:
    """The float64 oracle on the host copy of the same step: its append over the whole batch,
    then single-sequence decodes in order until the whole batch is done or ~budget_s passed."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    per_tok = 2 * w.num_kv_heads * w.head_dim * {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    L = w.lens_after_append
    t0 = time.perf_counter()
    ek, ev = oracle.reshape_and_cache(w.k_pool, w.v_pool, w.new_key, w.new_value, w.slot_mapping)
    seqs = done = 0
    # single-sequence decodes in batch order, cycling over the batch, until ~budget_s passed
    while seqs == 0 or time.perf_counter() - t0 < budget_s:
        b = seqs % w.batch
        sl = slice(b, b + 1)
        if window > 0:
            oracle.paged_decode_window(w.q[sl], ek, ev, w.block_table[sl], L[sl], w.scale, window)
            done += per_tok * min(int(L[b]), window)
        else:
            oracle.paged_decode(w.q[sl], ek, ev, w.block_table[sl], L[sl], w.scale)
            done += per_tok * int(L[b])
        seqs += 1
    dt = time.perf_counter() - t0
    return {"value": round(done / dt / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle", **_host_info(threads),
            "sample": f"oracle append of all {w.batch} tokens + float64 "
                      f"{'window-' + str(window) + ' ' if window > 0 else ''}decode of {seqs} sequences in batch "
                      f"order ({seqs / w.batch:.2f} passes over the batch; all heads, {done / 1e6:.1f} MB of KV) "
                      f"in {dt:.1f} s"}


def _cpu_baseline_beams(w, host, budget_s: float, window: int = 0) -> dict:
    """The float64 oracle on a host snapshot of one beam (all heads) of the 32K workload:
    its copy-on-write, its append and its decode, repeated until ~budget_s passed."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    L = np.full(1, w.context + 1, np.int32)
    per_seq = 2 * w.num_kv_heads * w.head_dim * 2 * (min(int(L[0]), window) if window > 0 else int(L[0]))
    t0 = time.perf_counter()
    reps = 0
    while reps == 0 or time.perf_counter() - t0 < budget_s:
        k1, v1 = oracle.copy_blocks(host["k_pool"], host["v_pool"], host["copy_pairs"])
        k2, v2 = oracle.reshape_and_cache(k1, v1, host["new_key"], host["new_value"], host["slot_mapping"])
        if window > 0:
            oracle.paged_decode_window(host["q"], k2, v2, host["table"], L, w.scale, window)
        else:
            oracle.paged_decode(host["q"], k2, v2, host["table"], L, w.scale)
        reps += 1
    dt = time.perf_counter() - t0
    return {"value": round(reps * per_seq / dt / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle", **_host_info(threads),
            "sample": f"{reps} x (copy-on-write + append + float64 "
                      f"{'window-' + str(window) + ' ' if window > 0 else ''}decode) of beam 0, all "
                      f"{w.num_kv_heads} heads, L={int(L[0])} ({per_seq / 1e6:.0f} MB of KV each) in {dt:.1f} s"}


def _cpu_baseline_fp8(w, budget_s: float, window: int = 0) -> dict:
    """The oracle's quantised step on host copies, one sequence at a time: its append of the
    new row into the sequence's (oracle-quantised) blocks, then its decode. Quantising the
    blocks that were already cached is setup and is not timed."""
    import oracle
    import oracle.fp8_cache as o8

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    per_tok = 2 * w.num_kv_heads * (w.head_dim + 4)
    L = w.lens_after_append
    bs = w.block_size
    timed = 0.0
    done = seqs = 0
    for b in range(w.batch):
        ids = w.block_table[b, :oracle.blocks_needed(int(L[b]), bs)]
        kc, ks = o8.quantize_rows(np.nan_to_num(w.k_pool[ids]))
        vc, vs = o8.quantize_rows(np.nan_to_num(w.v_pool[ids]))
        slot = int(w.slot_mapping[b])
        local = np.array([int(np.nonzero(ids == slot // bs)[0][0]) * bs + slot % bs], np.int32)
        table = np.arange(len(ids), dtype=np.int32)[None]
        t0 = time.perf_counter()
        pools = o8.reshape_and_cache_fp8(kc, vc, ks, vs, w.new_key[b:b + 1], w.new_value[b:b + 1], local)
        o8.paged_decode_fp8(w.q[b:b + 1], *pools, table, L[b:b + 1], w.scale, window=window)
        timed += time.perf_counter() - t0
        done += per_tok * (min(int(L[b]), window) if window > 0 else int(L[b]))
        seqs += 1
        if timed >= budget_s:
            break
    return {"value": round(done / timed / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle", **_host_info(threads),
            "sample": f"oracle quantised append + float64 {'window-' + str(window) + ' ' if window > 0 else ''}"
                      f"decode of sequences 0..{seqs - 1} (all heads, {done / 1e6:.1f} MB of codes and "
                      f"scales) in {timed:.1f} s"}


def _cpu_baseline_fp8_beams(w, host, budget_s: float, window: int = 0) -> dict:
    """The oracle's quantised step for one beam of the 32K workload, on the heads in ``host``."""
    import oracle.fp8_cache as o8

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    kc, ks = o8.quantize_rows(np.nan_to_num(host["k_pool"]))
    vc, vs = o8.quantize_rows(np.nan_to_num(host["v_pool"]))
    heads = host["k_pool"].shape[1]
    L = np.full(1, w.context + 1, np.int32)
    att = min(int(L[0]), window) if window > 0 else int(L[0])
    per_seq = 2 * heads * (w.head_dim + 4) * att
    t0 = time.perf_counter()
    reps = 0
    while reps == 0 or time.perf_counter() - t0 < budget_s:
        p1 = o8.copy_blocks_fp8(kc, vc, ks, vs, host["copy_pairs"])
        p2 = o8.reshape_and_cache_fp8(*p1, host["new_key"], host["new_value"], host["slot_mapping"])
        o8.paged_decode_fp8(host["q"], *p2, host["table"], L, w.scale, window=window)
        reps += 1
    dt = time.perf_counter() - t0
    return {"value": round(reps * per_seq / dt / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle", **_host_info(threads),
            "sample": f"{reps} x (quantised copy-on-write + append + float64 decode) of beam 0, "
                      f"{heads} of {w.num_kv_heads} heads, L={int(L[0])} in {dt:.1f} s"}


def _fp8_pools(kp, vp):
    """8-bit float copies of two float pools, quantised by the library's own append: every
    slot of the pool is appended once (unwritten NaN slots as zeros, never read)."""
    import torch

    from paged_kv_cache_indexed_amd import ops

    nb, hkv, bs, d = kp.shape
    k8, v8, ks, vs = ops.empty_fp8_cache(nb, hkv, bs, d, kp.device)
    slots = torch.arange(nb * bs, dtype=torch.int32, device=kp.device)

    def rows(x):
        return torch.nan_to_num(x).permute(0, 2, 1, 3).reshape(nb * bs, hkv, d).contiguous()

    ops.reshape_and_cache_fp8(rows(kp), rows(vp), k8, v8, ks, vs, slots)
    torch.cuda.synchronize()
    return k8, v8, ks, vs


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # MI355X dense matrix-core peak, published


def _timed(step, first: int, steps: int):
    """The timed region: `steps` steps with nothing else on the stream, bracketed by device
    synchronisation; returns the wall time in seconds."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(first + i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def _unique_slots(w, window: int) -> int:
    """Distinct physical (block, offset) slots the decode attends to over the whole batch: a
    slot shared by several sequences (a common prefix) counts once."""
    bs = w.block_size
    table = w.block_table if hasattr(w, "block_table") else w.table  # the beam workload's, after copy-on-write
    slots = []
    for b, L in enumerate(np.asarray(w.lens_after_append).tolist()):
        pos = np.arange(max(0, L - window) if window > 0 else 0, L, dtype=np.int64)
        slots.append(table[b, pos // bs].astype(np.int64) * bs + pos % bs)
    return int(np.unique(np.concatenate(slots)).size)


def _capture(fn, R: int) -> list:
    """fn(r) for r < R, each captured into its own HIP graph (the launches record their kernels
    on the capture stream; none of them allocates or clears memory)."""
    import torch

    graphs = []
    torch.cuda.synchronize()
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(r)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def _progress(msg: str) -> None:
    """One line on stderr per finished stage (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _host_info(threads: int) -> dict:
    """CPU model, the cores this process may run on and the numpy BLAS threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": blas,
            "threads_used": threads}


def _event_each(launch, first: int, steps: int) -> list:
    """Duration in us of each of `steps` launches, each between its own pair of HIP events on
    the launch stream (the event packets add a little to each figure)."""
    import torch

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        launch(first + i)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def _percentiles(xs) -> dict:
    v = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(v)), 2), "p10": round(float(np.percentile(v, 10)), 2),
            "p90": round(float(np.percentile(v, 90)), 2), "n": int(v.size)}


def _stream_ceiling(dev, gib: float = 4.0, reps: int = 10) -> dict:
    """Achievable streaming-read GB/s of this GPU: pa_measure_stream_read over `gib` GiB,
    8 work-groups per compute unit, `reps` back-to-back reads between one event pair."""
    import torch

    from paged_kv_cache_indexed_amd import _lib

    nbytes = int(gib * 2 ** 30)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wgs = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(wgs, dtype=torch.float32, device=dev)
    for _ in range(3):
        _lib.pa_measure_stream_read(buf, sink, wgs)
    ms = _event_pass(lambda i: _lib.pa_measure_stream_read(buf, sink, wgs), 0, reps)
    del buf, sink
    torch.cuda.empty_cache()
    return {"gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "workgroups": wgs,
            "kernel": "pa_measure_stream_read (16-byte non-temporal loads, 1 KiB per wave instruction)"}


def _sweep_config3(args, dev, medians=(87, 23), block_sizes=(8, 16, 32, 64)) -> dict:
    """The block-size sweep of the long-tail workload: for each median and block size, the
    fused step (pa_decode_append) timed as the main line is, the decode launch from the event
    pass, its share of the 8 TB/s roofline, and the padding waste."""
    import torch

    from paged_kv_cache_indexed_amd import _lib, ops
    from workloads import config3_device_family

    cases = {}
    for med in medians:
        fam = config3_device_family(med, block_sizes, dev)
        for w in fam:
            t = w.tensors
            pool_bytes = 2 * t["k_pool"].numel() * t["k_pool"].element_size()
            R = max(2, math.ceil(args.replica_bytes / pool_bytes))
            kps = [t["k_pool"]] + [t["k_pool"].clone() for _ in range(R - 1)]
            vps = [t["v_pool"]] + [t["v_pool"].clone() for _ in range(R - 1)]
            lens = t["lens_after"]
            max_len = int(w.lens_after_append.max())
            ws = ops.workspace_for(t["k_pool"], w.batch, w.num_q_heads, max_len, 0)
            out = torch.empty_like(t["q"])

            def step(i, kps=kps, vps=vps, t=t, lens=lens, max_len=max_len, ws=ws, out=out, w=w, R=R):
                ops.decode_append(t["q"], kps[i % R], vps[i % R], t["block_table"], lens, max_len, w.scale,
                                  t["new_key"], t["new_value"], t["slot_mapping"], out=out, workspace=ws)

            for i in range(args.warmup):
                step(i)
            wall = _timed(step, args.warmup, args.steps)
            dec = _event_pass(step, args.warmup + args.steps, args.steps)
            gat = _gather_ms(args, w, t, kps, vps, R)
            kv = 2 * w.num_kv_heads * w.head_dim * 2 * int(w.lens_after_append.sum())
            gbs = kv / (dec * 1e-3) / 1e9
            part = _lib.pa_decode_partition_size(_lib.CacheDesc.of(t["k_pool"]), w.batch, w.num_q_heads, max_len, 0)
            _progress(f"sweep median {med} block size {w.block_size}: decode {dec * 1e3:.1f} us")
            cases[f"med{med}-bs{w.block_size}"] = {
                "decode_launch_us": round(dec * 1e3, 2), "decode_gbs": round(gbs, 1),
                "frac": round(gbs / HBM_PEAK_GBS, 4), "gather_us": round(gat * 1e3, 2),
                "frac_of_gather": round(gat / dec, 4), "step_us": round(wall * 1e6 / args.steps, 2),
                "step_gbs": round(kv / (wall / args.steps) / 1e9, 1), "kv_bytes": kv,
                "context_len_sum": int(w.lens_after_append.sum()), "context_len_max": max_len,
                "partition_size": part, "replicas": R,
                "padding_waste_pct": round(padding_waste_pct(w.lens_after_append, w.block_size), 2)}
            del kps, vps, t, ws, out, step
        del fam
        torch.cuda.empty_cache()
    worst = min(cases, key=lambda k: cases[k]["frac"])
    return {"workload": "cfg3-f16-longtail, fused step (append + decode), cold replicas",
            "cases": cases, "worst": {"case": worst, "frac": cases[worst]["frac"]},
            "all_at_least_70pct": all(c["frac"] >= 0.70 for c in cases.values())}


def _gather_ms(args, w, t, kps, vps, R: int) -> float:
    """Average duration in ms of pa_measure_gather_read over the step's replicas: the split
    decode's reads of this cache (K and V below the lengths, through the table) alone."""
    import torch

    from paged_kv_cache_indexed_amd import _lib

    lens = t["lens_after"]
    max_len = int(w.lens_after_append.max())
    sink = torch.empty(w.batch * w.num_kv_heads, dtype=torch.float32, device=lens.device)
    desc = _lib.CacheDesc.of(t["k_pool"])

    def gather(i):
        _lib.pa_measure_gather_read(desc, kps[i % R], vps[i % R], t["block_table"], lens, max_len, sink)

    for i in range(args.warmup):
        gather(i)
    return _event_pass(gather, args.warmup, args.steps)


def _config1_line(args, dev) -> dict:
    """Config 1, the tiny fp32 workload (4 sequences, 1.3 MB of K+V): the fused step and its
    decode launch timed as the main line is, the launch's share of the 8 TB/s roofline, and
    the oracle on the host (a few seconds). At this size a launch is its fixed costs."""
    import torch

    from paged_kv_cache_indexed_amd import _lib, ops

    w = _workload(1, None, None)
    t = w.to_device(dev)
    pool_bytes = 2 * t["k_pool"].numel() * t["k_pool"].element_size()
    R = max(2, math.ceil(args.replica_bytes / pool_bytes))
    kps = [t["k_pool"]] + [t["k_pool"].clone() for _ in range(R - 1)]
    vps = [t["v_pool"]] + [t["v_pool"].clone() for _ in range(R - 1)]
    lens = t["lens_after"]
    max_len = int(w.lens_after_append.max())
    ws = ops.workspace_for(t["k_pool"], w.batch, w.num_q_heads, max_len, 0)
    out = torch.empty_like(t["q"])

    def step(i):
        ops.decode_append(t["q"], kps[i % R], vps[i % R], t["block_table"], lens, max_len, w.scale,
                          t["new_key"], t["new_value"], t["slot_mapping"], out=out, workspace=ws)

    for i in range(args.warmup):
        step(i)
    wall = _timed(step, args.warmup, args.steps)
    dec = _event_pass(step, args.warmup + args.steps, args.steps)
    kv = 2 * w.num_kv_heads * w.head_dim * 4 * int(w.lens_after_append.sum())
    gbs = kv / (dec * 1e-3) / 1e9
    _progress(f"config 1: decode {dec * 1e3:.1f} us")
    line = {"workload": w.name, "decode_launch_us": round(dec * 1e3, 2), "decode_gbs": round(gbs, 2),
            "frac": round(gbs / HBM_PEAK_GBS, 5), "step_us": round(wall * 1e6 / args.steps, 2),
            "kv_bytes": kv, "decode_tokens_per_s": round(w.batch / wall * args.steps, 1), "replicas": R,
            "partition_size": _lib.pa_decode_partition_size(_lib.CacheDesc.of(t["k_pool"]), w.batch,
                                                            w.num_q_heads, max_len, 0)}
    del kps, vps
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(w, min(3.0, args.cpu_budget))
    return line


def _event_pass(launch, first: int, steps: int) -> float:
    """Average duration in ms of the measured kernel: `steps` back-to-back launches of it (same
    inputs and replica rotation as the steps) between one pair of HIP events on its stream.
    An event pair around every single launch would add 2-5 us to each measured duration."""
    import torch

    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        launch(first + i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _bench_multi(args, dev) -> int:
    """Multi-token step: N new tokens per sequence appended after the workload's context, then
    pa_multi_token_attention of those N causal queries over the grown context (with --kv fp8
    over 8-bit pools, appended by the quantising append)."""
    import torch

    from paged_kv_cache_indexed_amd import _lib, ops
    from workloads import build_paged

    N = int(args.queries)
    base = _workload(args.config, args.block_size, args.median)
    if base.dtype not in ("f16", "bf16"):
        print("--queries needs a workload with fp16 or bf16 pools", file=sys.stderr)
        return 2
    lens = (base.context_lens + N).astype(np.int32)
    w = build_paged(f"{base.name}-q{N}", base.meta["cfg"], 0, lens, base.block_size, base.num_kv_heads,
                    base.num_q_heads, base.head_dim, base.dtype, scale=base.scale, std=base.meta["std"],
                    append=False)
    t = w.to_device(dev)
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    qs = np.arange(B + 1, dtype=np.int32) * N
    gen = torch.Generator(device=dev).manual_seed(11)
    q = torch.randn((B * N, Hq, d), generator=gen, device=dev).to(t["k_pool"].dtype)
    kc, vc, starts = w.meta["contents_k"], w.meta["contents_v"], w.meta["starts"]
    rows = np.concatenate([np.arange(L - N, L) + starts[b] for b, L in enumerate(lens)])
    keys = torch.from_numpy(kc[rows]).to(t["k_pool"].dtype).to(dev)
    vals = torch.from_numpy(vc[rows]).to(t["k_pool"].dtype).to(dev)
    tok = np.concatenate([np.arange(L - N, L) for L in lens])
    seq = np.repeat(np.arange(B), N)
    slots = torch.from_numpy((w.block_table[seq, tok // w.block_size] * w.block_size + tok % w.block_size)
                             .astype(np.int32)).to(dev)
    fp8 = args.kv == "fp8"
    if fp8:
        pools = _fp8_pools(t["k_pool"], t["v_pool"])
        del t["k_pool"], t["v_pool"]
    else:
        pools = (t["k_pool"], t["v_pool"], None, None)
    pool_bytes = sum(x.numel() * x.element_size() for x in pools if x is not None)
    R = max(2, math.ceil(args.replica_bytes / pool_bytes))
    reps = [pools] + [tuple(x.clone() if x is not None else None for x in pools) for _ in range(R - 1)]
    qs_d = torch.from_numpy(qs).to(dev)
    max_len = int(lens.max())
    desc = _lib.CacheDesc.of(pools[0])
    wsn = _lib.pa_multi_token_workspace_bytes(desc, B, B * N, Hq, max_len, N, args.partition_size)
    ws = torch.empty((wsn + 3) // 4, dtype=torch.float32, device=dev) if wsn else None
    out = torch.empty_like(q)
    def attend(i):
        kp, vp, ks, vs = reps[i % R]
        ops.multi_token_attention(q, kp, vp, t["block_table"], t["context_lens"], qs_d, max_len, N, w.scale,
                                  k_scale=ks, v_scale=vs, partition_size=args.partition_size, out=out, workspace=ws)

    def step(i):
        kp, vp, ks, vs = reps[i % R]
        if fp8:
            ops.reshape_and_cache_fp8(keys, vals, kp, vp, ks, vs, slots)
        else:
            ops.reshape_and_cache(keys, vals, kp, vp, slots)
        attend(i)

    for i in range(args.warmup):
        step(i)
    wall = _timed(step, args.warmup, args.steps)
    ms = _event_pass(attend, args.warmup + args.steps, args.steps)
    row_bytes = d + 4 if fp8 else d * q.element_size()  # codes + scale, or elements
    kv_bytes = 2 * w.num_kv_heads * row_bytes * int(lens.sum())
    visible = sum(int((L - N + np.arange(N) + 1).sum()) for L in lens)  # (query, key) pairs per head
    flops = 4.0 * Hq * d * visible
    sec = ms * 1e-3
    gbs, tfl = kv_bytes / sec / 1e9, flops / sec / 1e12
    peak_t = MFMA_PEAK_TFLOPS[w.dtype]
    mfma_bound = flops / kv_bytes > peak_t * 1e12 / (HBM_PEAK_GBS * 1e9)
    cfg = _describe(w)
    if fp8:
        cfg["workload"] = f"{w.name}-fp8"
    cfg.update({"queries_per_seq": N, "replicas": R,
                "step": f"append {N} tokens/seq + causal attention of those {N} queries"})
    result = {
        "metric": "multi-token paged attention: query tokens/s at 1 MI355X",
        "value": round(B * N / (wall / args.steps), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": f"e4m3+{w.dtype}" if fp8 else w.dtype,
        "data": "synthetic", "config": cfg, "attention_kernel_ms": round(ms, 5),
        "kv_gbs": round(gbs, 1), "tflops": round(tfl, 2),
        "roofline": ({"bound": "mfma", "achieved": round(tfl, 2), "peak": peak_t, "unit": "TFLOP/s",
                      "frac": round(tfl / peak_t, 4), "traffic": None} if mfma_bound else
                     {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}),
        "kernel_source_hash": kernel_source_hash("multi"),
        "mfma_busy_pct": recorded_mfma_busy(cfg["workload"], "multi"),
    }
    if not args.no_cpu_baseline:
        import oracle

        t1 = time.perf_counter()
        done = nseq = 0
        while nseq < B and (nseq == 0 or time.perf_counter() - t1 < args.cpu_budget):
            sl = slice(nseq, nseq + 1)
            oracle.paged_attention_multi(q[nseq * N:(nseq + 1) * N].float().cpu().numpy(), w.k_pool, w.v_pool,
                                         w.block_table[sl], lens[sl], np.array([0, N]), w.scale)
            done += N
            nseq += 1
        dt = time.perf_counter() - t1
        try:
            from threadpoolctl import threadpool_info
            threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
        except Exception:  # noqa: BLE001
            threads = 1
        result["cpu_baseline"] = {"value": round(done / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle", **_host_info(threads),
                                  "sample": f"float64 multi-token attention of sequences 0..{nseq - 1} "
                                            f"({done} query tokens, all heads) in {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def _bench_reblock(args, w, t, kps, vps, R, dev) -> int:
    """Time pa_reblock of the workload's cache (context_lens tokens per sequence) into a new
    layout of block size args.reblock; bytes = the valid K+V rows read plus written."""
    import torch

    from paged_kv_cache_indexed_amd import ops

    if args.kv == "fp8":
        print("--reblock times 16/32-bit pools only", file=sys.stderr)
        return 2
    nbs = int(args.reblock)
    lens_np = w.context_lens
    need = -(-lens_np // nbs)
    nnb = int(need.sum())
    perm = np.random.default_rng([7, nbs]).permutation(nnb).astype(np.int32)
    ntab = np.full((w.batch, int(need.max())), -1, np.int32)
    cur = 0
    for b, n in enumerate(need.tolist()):
        ntab[b, :n] = perm[cur:cur + n]
        cur += n
    shape = (nnb,) + tuple(t["k_pool"].shape[1:2]) + (nbs,) + tuple(t["k_pool"].shape[3:])
    dk = torch.empty(shape, dtype=kps[0].dtype, device=dev)
    dv = torch.empty_like(dk)
    ntab_d = torch.from_numpy(ntab).to(dev)
    lens = t["context_lens"]
    max_len = int(lens_np.max())
    moved = 2 * 2 * w.num_kv_heads * w.head_dim * kps[0].element_size() * int(lens_np.sum())
    stream = torch.cuda.current_stream()
    def step(i):
        ops.reblock(kps[i % R], vps[i % R], t["block_table"], dk, dv, ntab_d, lens, max_len)

    for i in range(args.warmup):
        step(i)
    wall = _timed(step, args.warmup, args.steps)
    ms = _event_pass(step, args.warmup + args.steps, args.steps)
    achieved = moved / (ms * 1e-3) / 1e9
    cfg = _describe(w)
    cfg.update({"workload": f"{w.name}-reblock{w.block_size}to{nbs}", "new_block_size": nbs, "replicas": R,
                "step": "pa_reblock of every valid K/V row to the new layout"})
    print(json.dumps({
        "metric": "re-blocking GB/s (valid K+V rows read + written) at 1 MI355X",
        "value": round(moved / (wall / args.steps) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic", "config": cfg,
        "kernel_ms": round(ms, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1-5 (default 3: the long-tail lengths, median 87, block size 16)")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--median", type=float, default=None)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--kv", choices=["native", "fp8"], default="native",
                    help="pool elements: the workload's dtype, or 8-bit floats with a scale per row")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per replica instead of launching from Python")
    ap.add_argument("--beams", type=int, default=None,
                    help="decode with pa_decode_beams, sequences grouped by this many beams (append separate); "
                         "config 5 defaults to its beam width (4), --beams 0 decodes with pa_decode_append")
    ap.add_argument("--contiguous-pool", action="store_true",
                    help="configs 2-4: each sequence's blocks consecutive in id order (same lengths and contents), "
                         "to measure what scattered blocks and their table lookups cost")
    ap.add_argument("--unfused", action="store_true",
                    help="append with pa_reshape_and_cache and decode with pa_decode (two launches)")
    ap.add_argument("--queries", type=int, default=0,
                    help="multi-token step: append this many tokens per sequence, then their causal attention")
    ap.add_argument("--layers", type=int, default=1,
                    help="run the step on one layer's strided view of a [blocks][2][layers][heads][bs][d] cache")
    ap.add_argument("--reblock", type=int, default=0,
                    help="instead of the step, time pa_reblock of the cache to this block size")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: attend to the last W tokens only (0: whole context)")
    ap.add_argument("--replica-bytes", type=float, default=1.5 * 2 ** 30,
                    help="pool bytes touched between reuses of one replica")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the block-size x median sweep that accompanies the default workload")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--variant", action="store_true",
                    help="allow PAGEDKV_LIB to name a library other than the in-tree build")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    if os.environ.get("PAGEDKV_LIB") and not args.variant:
        print("PAGEDKV_LIB is set: bench.py measures the in-tree library unless --variant is given",
              file=sys.stderr)
        return 2
    if args.config == 3 and args.median is None:
        args.median = 87
    if args.contiguous_pool and args.config not in (2, 3, 4):
        print("--contiguous-pool applies to configs 2-4", file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_indexed_amd import _lib, ops

    _lib.load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    if args.queries > 0:
        return _bench_multi(args, dev)
    host_sample = None
    if args.config == 5:
        from workloads.longctx import beam_workload, host_subset

        w = beam_workload(dev)
        t = dict(w.tensors)
        if not args.no_cpu_baseline:
            host_sample = host_subset(w, [0], range(4 if args.kv == "fp8" else w.num_kv_heads))
    else:
        w = _workload(args.config, args.block_size, args.median, args.contiguous_pool)
        t = w.to_device(dev)
        _progress(f"{w.name}: workload on the device")
    fp8 = args.kv == "fp8"
    if fp8 and w.dtype == "f32":
        print("--kv fp8 needs a workload with fp16 or bf16 queries", file=sys.stderr)
        return 2
    if fp8:
        k8, v8, ks8, vs8 = _fp8_pools(t["k_pool"], t["v_pool"])
        t["k_pool"], t["v_pool"] = k8, v8
        pool_bytes = 2 * (k8.numel() + 4 * ks8.numel())
    else:
        pool_bytes = 2 * t["k_pool"].numel() * t["k_pool"].element_size()
    NL = max(1, args.layers)
    R = max(2, math.ceil(args.replica_bytes / (pool_bytes * NL)))
    if NL > 1:
        # one allocation per replica holding NL layers' K and V; the step reads the last layer
        def layered(kp, vp):
            cache = torch.zeros((kp.shape[0], 2, NL) + tuple(kp.shape[1:]), dtype=kp.dtype, device=dev)
            cache[:, 0, NL - 1].copy_(kp)
            cache[:, 1, NL - 1].copy_(vp)
            return cache
        caches = [layered(t["k_pool"], t["v_pool"]) for _ in range(R)]
        kps = [c[:, 0, NL - 1] for c in caches]
        vps = [c[:, 1, NL - 1] for c in caches]
    else:
        kps = [t["k_pool"]] + [t["k_pool"].clone() for _ in range(R - 1)]
        vps = [t["v_pool"]] + [t["v_pool"].clone() for _ in range(R - 1)]
    if fp8:
        kss = [ks8] + [ks8.clone() for _ in range(R - 1)]
        vss = [vs8] + [vs8.clone() for _ in range(R - 1)]
    lens = t["lens_after"]
    max_len = int(w.lens_after_append.max())
    P = args.partition_size
    W = max(0, args.window)
    if args.beams is None:
        args.beams = w.beams if args.config == 5 and W <= 0 else 0
    BW = max(0, args.beams)
    if BW and W > 0:
        print("--beams has no window", file=sys.stderr)
        return 2
    if BW:
        nws = _lib.pa_decode_beams_workspace_bytes(_lib.CacheDesc.of(t["k_pool"]), w.batch, BW, w.num_q_heads,
                                                   max_len, P)
        ws = torch.empty((nws + 3) // 4, dtype=torch.float32, device=dev) if nws else None
    else:
        ws = ops.workspace_for(t["k_pool"], w.batch, w.num_q_heads, max_len, P, window=W)
    out = torch.empty_like(t["q"])
    pairs = t["copy_pairs"]
    esize = t["k_pool"].element_size()
    attended = np.minimum(w.lens_after_append, W) if W > 0 else w.lens_after_append
    row_bytes = w.head_dim + 4 if fp8 else w.head_dim * esize  # codes + scale, or elements
    kv_bytes = 2 * w.num_kv_heads * row_bytes * int(attended.sum())
    stream = torch.cuda.current_stream()

    # append and decode fused unless a window or beam groups are set, or asked not to
    fused = not (W > 0 or args.unfused or BW)

    def decode(i):  # the measured kernel: the decode launch of step i
        r = i % R
        if BW:
            ops.decode_beams(t["q"], kps[r], vps[r], t["block_table"], lens, max_len, w.scale, BW,
                             k_scale=kss[r] if fp8 else None, v_scale=vss[r] if fp8 else None, partition_size=P,
                             out=out, workspace=ws)
        elif fused and fp8:
            ops.decode_append_fp8(t["q"], kps[r], vps[r], kss[r], vss[r], t["block_table"], lens, max_len, w.scale,
                                  t["new_key"], t["new_value"], t["slot_mapping"], partition_size=P, out=out,
                                  workspace=ws)
        elif fused:
            ops.decode_append(t["q"], kps[r], vps[r], t["block_table"], lens, max_len, w.scale, t["new_key"],
                              t["new_value"], t["slot_mapping"], partition_size=P, out=out, workspace=ws)
        elif fp8:
            ops.decode_fp8(t["q"], kps[r], vps[r], kss[r], vss[r], t["block_table"], lens, max_len, w.scale,
                           window=W, partition_size=P, out=out, workspace=ws)
        else:
            ops.decode(t["q"], kps[r], vps[r], t["block_table"], lens, max_len, w.scale,
                       partition_size=P, out=out, workspace=ws, window=W)

    def step(i):
        r = i % R
        if fp8:
            if pairs.shape[0]:
                ops.copy_blocks_fp8(kps[r], vps[r], kss[r], vss[r], pairs)
            if not fused:
                ops.reshape_and_cache_fp8(t["new_key"], t["new_value"], kps[r], vps[r], kss[r], vss[r],
                                          t["slot_mapping"])
        else:
            if pairs.shape[0]:
                ops.copy_blocks(kps[r], vps[r], pairs)
            if not fused:
                ops.reshape_and_cache(t["new_key"], t["new_value"], kps[r], vps[r], t["slot_mapping"])
        decode(i)

    if args.calib_copy_mb > 0:
        nbytes = args.calib_copy_mb << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.reblock:
        return _bench_reblock(args, w, t, kps, vps, R, dev)
    for i in range(args.warmup):
        step(i)
    run_step, run_decode = step, decode
    if args.graph:
        # One HIP graph per replica for the step and for the decode launch alone. Measured
        # 3-12% slower than launching from Python on every workload here (the Python and
        # ctypes time of a launch hides behind the kernel before it), so not the default.
        step_g, dec_g = _capture(step, R), _capture(decode, R)
        run_step, run_decode = (lambda i: step_g[i % R].replay()), (lambda i: dec_g[i % R].replay())
        for i in range(2 * R):
            run_step(i)
    _progress(f"{w.name}: warm-up done")
    wall = _timed(run_step, args.warmup, args.steps)
    dec_avg = _event_pass(run_decode, args.warmup + args.steps, args.steps)
    _progress(f"{w.name}: {wall * 1e6 / args.steps:.1f} us per step, decode launch {dec_avg * 1e3:.1f} us")
    dec_each = _event_each(run_decode, args.warmup + 2 * args.steps, args.steps)
    step_each = _event_each(run_step, args.warmup + 3 * args.steps, args.steps)
    ms_step = wall * 1e3 / args.steps
    # Blocks shared by several sequences (beams of one prompt) hold one copy of their bytes:
    # the roofline counts each attended physical slot once, the least the launch has to move.
    roof_bytes = 2 * w.num_kv_heads * row_bytes * _unique_slots(w, W)
    achieved = roof_bytes / (dec_avg * 1e-3) / 1e9
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    path = ("beams" if BW else
            decode_path("fp8" if fp8 else w.dtype, w.head_dim, w.num_q_heads // w.num_kv_heads, w.block_size))
    span = min(max_len, W + w.block_size - 1) if W > 0 else max_len
    if BW:
        part = _lib.pa_decode_beams_partition_size(_lib.CacheDesc.of(t["k_pool"]), w.batch, BW, w.num_q_heads,
                                                   max_len, P)
    else:
        part = _lib.pa_decode_partition_size(_lib.CacheDesc.of(t["k_pool"]), w.batch, w.num_q_heads, span, P)
    cfg = _describe(w)
    if NL > 1:
        cfg["workload"] = f"{w.name}-layer{NL - 1}of{NL}"
        cfg["block_stride_bytes"] = int(kps[0].stride(0) * kps[0].element_size())
    if fp8:
        cfg["workload"] = f"{cfg['workload']}-fp8"
        cfg["kv_storage"] = "OCP E4M3 codes + float32 scale per (token, kv head) row"
    if W > 0:
        cfg["workload"] = f"{cfg['workload']}-window{W}"
        cfg["window"] = W
        cfg["attended_tokens_sum"] = int(attended.sum())
    cfg.update({"partition_size": part, "replicas": R, "tokens_per_step": w.batch,
                "launch": "hip graph per replica" if args.graph else "eager",
                "copy_pairs_per_step": int(pairs.shape[0]),
                "step": ("copy-on-write + " if pairs.shape[0] else "") + "append 1 token/seq + decode"
                        + (" (append fused into the decode: pa_decode_append)" if fused else "")
                        + (f" (pa_decode_beams, groups of {BW} beams)" if BW else "")})
    if BW:
        cfg["workload"] = f"{cfg['workload']}-beamdecode{BW}"
    if roof_bytes != kv_bytes:
        cfg["roofline_bytes"] = roof_bytes  # unique K+V bytes: shared blocks counted once
    if args.config == 5:
        cfg["unique_kv_bytes"] = 2 * w.unique_blocks * w.block_size * w.num_kv_heads * row_bytes
    result = {
        "metric": "paged-decode KV GB/s (% of HBM peak) and decode tokens/s at 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"e4m3+{w.dtype}" if fp8 else w.dtype,
        "data": "synthetic (seeded N(0,1) contents, shuffled physical pool, NaN-filled padding)",
        "config": cfg,
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
        "decode_kernel_ms": round(dec_avg, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(cfg["workload"], path),
                     "algorithmic_bytes": int(roof_bytes)},
        "kernel_source_hash": kernel_source_hash(path),
        "decode_kernel": path,
        "decode_launch_us_per_launch_events": _percentiles(dec_each),
        "step_us_per_step_events": _percentiles(step_each),
        "library": _lib.library_identity(),
    }
    if not args.no_ceiling:
        ceil = _stream_ceiling(dev)
        result["roofline"]["ceiling"] = ceil["gbs"]
        result["roofline"]["frac_of_ceiling"] = round(achieved / ceil["gbs"], 4)
        result["stream_read_ceiling"] = ceil
    if not (fp8 or W or BW or NL > 1):
        # the same cache read by the split decode's loads alone, in its decomposition
        gat = _gather_ms(args, w, t, kps, vps, R)
        result["roofline"]["gather_ceiling"] = round(roof_bytes / (gat * 1e-3) / 1e9, 1)
        result["roofline"]["frac_of_gather_ceiling"] = round(gat / dec_avg, 4)
    plain = not (fp8 or W or BW or args.unfused or args.graph or NL > 1 or args.contiguous_pool)
    if args.config == 3 and plain and not args.no_sweep:
        del kps, vps
        torch.cuda.empty_cache()
        result["sweep"] = _sweep_config3(args, dev)
        result["config1"] = _config1_line(args, dev)
    if path == "mfma":
        result["mfma_busy_pct"] = recorded_mfma_busy(cfg["workload"], path)
    if not args.no_cpu_baseline:
        _progress("oracle timing on the host")
        if fp8:
            result["cpu_baseline"] = (_cpu_baseline_fp8_beams(w, host_sample, args.cpu_budget, W) if host_sample
                                      else _cpu_baseline_fp8(w, args.cpu_budget, W))
        else:
            result["cpu_baseline"] = (_cpu_baseline_beams(w, host_sample, args.cpu_budget, W) if host_sample
                                      else _cpu_baseline(w, args.cpu_budget, W))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
