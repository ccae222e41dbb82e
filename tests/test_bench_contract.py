"""bench.py's output contract: one JSON line with the metric, the roofline of the decode
launch and the oracle timed on the host (GPU), and the refusal of several GPUs (CPU)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600, env=None):
    return subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout, env=env)


def test_bench_refuses_another_library_unless_asked():
    env = dict(os.environ, PAGEDKV_LIB="/nonexistent/libpagedkv.so")
    r = _bench("--steps", "1", timeout=120, env=env)
    assert r.returncode == 2 and "PAGEDKV_LIB" in r.stderr and r.stdout.strip() == ""


def test_bench_refuses_several_gpus():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_default_line():
    print("[gpu-case] bench.py default workload, 3 steps, no sweep", flush=True)
    r = _bench("--steps", "3", "--warmup", "1", "--cpu-budget", "1", "--no-sweep")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key, kind in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[key], kind), key
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["unit"] == "GB/s"
    assert "synthetic" in d["data"]
    cfg = d["config"]
    assert isinstance(cfg["workload"], str) and cfg["workload"]
    # value is the effective K+V bytes of the step over its time
    step_bytes = 2 * cfg["num_kv_heads"] * cfg["head_dim"] * 2 * cfg["context_len_sum"]
    assert d["value"] * d["ms_per_step"] * 1e6 == pytest.approx(step_bytes, rel=2e-3)
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert roof["traffic"] is None or (isinstance(roof["traffic"], int) and roof["traffic"] > 0)
    # achieved is the algorithmic bytes of one decode launch over its average duration
    assert roof["algorithmic_bytes"] == step_bytes
    assert roof["achieved"] * d["decode_kernel_ms"] * 1e6 == pytest.approx(step_bytes, rel=2e-3)
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["unit"]
    assert isinstance(cpu["sample"], str) and cpu["sample"]
    assert cpu["cpu_model"] and cpu["affinity_cores"] >= 1
    assert cfg["workload"].startswith("cfg3-f16-longtail-med87-bs16")
    assert roof["ceiling"] > 1000 and roof["frac_of_ceiling"] == pytest.approx(roof["achieved"] / roof["ceiling"],
                                                                                 abs=1e-3)
    # the same cache's reads alone: at least as fast as the decode that also computes on them,
    # within launch-to-launch noise
    assert roof["gather_ceiling"] > 1000 and 0 < roof["frac_of_gather_ceiling"] < 1.15
    lib = d["library"]
    assert lib["in_tree"] is True and len(lib["sha256_16"]) == 16
    for k in ("decode_launch_us_per_launch_events", "step_us_per_step_events"):
        p = d[k]
        assert p["p10"] <= p["median"] <= p["p90"] and p["n"] == 3
