"""bench.py's command-line contract: it runs on one GPU only and says so for
--gpus N > 1, and it refuses conflicting modes, both before any GPU work (CPU
tests); on a GPU, its JSON line carries the report keys."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_conflicting_modes_are_refused():
    r = run("--stats", "--lse-in")
    assert r.returncode == 2
    assert "separate modes" in r.stderr


@pytest.mark.gpu
def test_bench_line_carries_the_report_keys():
    """One bench line on the small fp32 workload: the spread of the step
    times, the launch form, the cache-flush flag, the roofline object and the
    CPU baseline with its core count and CPU model."""
    import json

    r = run("--workload", "tiny_f32_2k", "--steps", "5", "--warmup", "2")
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "ms_per_step", "ms_per_step_median", "ms_per_step_min",
                "ms_per_step_max", "stage_ms", "roofline", "cpu_baseline", "config"):
        assert key in line, key
    assert line["ms_per_step_min"] <= line["ms_per_step_median"] <= line["ms_per_step_max"]
    assert line["config"]["workload"] == "tiny_f32_2k"
    assert line["config"]["launch"] == "hip graph"
    assert line["config"]["cache_flush_between_steps"] is True   # 1 MiB of K
    roof = line["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    cpu = line["cpu_baseline"]
    assert cpu["cores"] >= 1 and cpu["kind"] == "oracle" and isinstance(cpu["cpu_model"], str)


@pytest.mark.gpu
@pytest.mark.parametrize("mode,flushed", [("--decode", True), ("--csm", False), ("--stats", False),
                                          ("--lse-in", False), ("--max-pool", False)])
def test_bench_other_modes_run(mode, flushed):
    """Each of the other bench modes prints one JSON line with its roofline
    (short runs, no CPU baseline) and says whether a cache flush ran between
    its timed calls: the decode cache (268 MB) is flushed, the CSM inputs
    (1 GiB) and the 128K workload's K (4.3 GB) are not."""
    import json

    r = run(mode, "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["value"] > 0 and line["roofline"]["frac"] > 0
    assert line["config"]["cache_flush_between_steps"] is flushed
    if mode == "--max-pool":
        assert line["config"]["pool_type"] == "max"


@pytest.mark.gpu
@pytest.mark.parametrize("workload,extra", [("llama8b_32k_tsp", ()), ("llama8b_32k_tsp", ("--no-graph",)),
                                            ("batched_8x32k_ar1", ()), ("batched_8x32k_ar1", ("--stats",)),
                                            ("batched_8x32k_ar1", ("--max-pool",))])
def test_bench_concurrent_step_matches_serial(workload, extra):
    """The timed step (the token-set chain beside the per-head top-k on a
    second stream where the workload has one), replayed from a HIP graph or
    launched each step: every output must equal a serial eager step's, byte
    for byte."""
    import json

    r = run("--workload", workload, *extra, "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--check")
    assert r.returncode == 0, (r.stdout[-1000:], r.stderr[-2000:])
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["check"] == "identical"
    assert line["config"]["token_set_chain"] == ("beside the per-head top-k" if workload.startswith("llama") else None)
