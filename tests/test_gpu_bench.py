"""bench.py's output on the GPU: one JSON line per run, with every key of its
contract (metric, value, unit, n_gpus, steps, warmup, ms_per_step,
higher_is_better, scaling, vs_baseline, dtype, data, config with the
workload, roofline with bound / achieved / peak / unit / frac / traffic, and
cpu_baseline when the oracle leg runs).  Each run is a short child process;
the numbers are only checked for sense, not for speed."""

import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def bench_line(*args, timeout=240):
    # device_count() does not initialise the GPU in this process: the child
    # process is the only one here that uses it
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    print(f"[gpu] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_common(d, steps, warmup):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["unit"] == "tokens/s" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None and d["data"] == "synthetic"
    assert isinstance(d["config"].get("workload"), str)
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert 0 < rl["achieved"] < rl["peak"] and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert "traffic" in rl


def test_prefill_line_with_the_oracle_leg():
    """The smallest workload, the oracle leg included: tokens/s is whole-job
    throughput, B*T / ms_per_step."""
    d = bench_line("--workload", "1", "--steps", "3", "--warmup", "2")
    check_common(d, 3, 2)
    assert d["dtype"] == "bf16"
    cfg = d["config"]
    # ms_per_step is printed to 4 decimals: the rate recomputed from it may be
    # off by that rounding, relative 5e-5 / ms_per_step
    tol = d["value"] * 6e-5 / d["ms_per_step"] + 1.0
    assert abs(d["value"] - cfg["n_tokens"] / (d["ms_per_step"] / 1e3)) <= tol
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["unit"] == "tokens/s"
    assert cpu["cores"] >= 1 and cpu["host_cores"] >= 1 and isinstance(cpu["sample"], str)
    assert set(d["kernels"]) == {"chunk_cumsum_recompute_wu", "chunk_delta_h_fwd_o"}


def test_decode_line():
    d = bench_line("--decode", "--steps", "3", "--warmup", "2", "--no-cpu-baseline")
    check_common(d, 3, 2)
    assert d["config"]["workload"] == "decode_B256" and d["cpu_baseline"] is None
    assert d["roofline"]["kernel"] == "recurrent_decode"
