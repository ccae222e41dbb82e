import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size configuration (minutes of host work)")


def pytest_report_header(config):
    """Name the HIP library the tests load (path, hash, in-tree or not)."""
    try:
        from paged_kv_cache_indexed_amd import _lib

        ident = _lib.library_identity()
        return [f"libpagedkv: {ident['path']} sha256 {ident['sha256_16']} in_tree={ident['in_tree']}"]
    except Exception as e:  # noqa: BLE001 - a missing library is reported by the tests themselves
        return [f"libpagedkv: not loaded ({type(e).__name__}: {e})"]


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """After a GPU run: the library loaded, and every parity comparison's raw max-abs error
    against the literal bound (1e-5 fp32, 2e-3 fp16, 1e-2 bf16) and against the bound plus
    half an ulp of the output (the test criterion)."""
    import sys

    gu = sys.modules.get("tests.gpu_util")
    if gu is None or not gu.RESULTS:
        return
    tr = terminalreporter
    try:
        from paged_kv_cache_indexed_amd import _lib

        ident = _lib.library_identity()
        tr.write_line(f"libpagedkv: {ident['path']} sha256 {ident['sha256_16']} in_tree={ident['in_tree']}")
    except Exception:  # noqa: BLE001
        pass
    rows = gu.RESULTS
    literal = [r for r in rows if r[2] <= gu.TOL[r[1]]]
    tr.write_line(f"parity: {len(rows)} comparisons vs the oracle; raw max-abs within the literal bound in "
                  f"{len(literal)}; within bound + output half-ulp in "
                  f"{sum(1 for r in rows if r[3] <= gu.TOL[r[1]])}")
    for dt in ("f32", "f16", "bf16"):
        sub = [r for r in rows if r[1] == dt]
        if sub:
            worst = max(sub, key=lambda r: r[2] / gu.TOL[dt])
            tr.write_line(f"parity {dt}: {len(sub)} cases, worst raw max-abs {worst[2]:.3e} "
                          f"(bound {gu.TOL[dt]:.0e}) in '{worst[0]}'")
    for r in rows:
        if r[2] > gu.TOL[r[1]]:
            tr.write_line(f"parity beyond the literal bound only by output rounding: '{r[0]}' raw {r[2]:.3e}, "
                          f"beyond rounding {r[3]:.3e}")
