"""The four bf16 workloads at their full sizes, in the launch configuration
the benchmark times (one scoring call over every layer), against the fp64
oracle on every score, LSE, kept index and gathered row."""

import time

import numpy as np

import pytest

from gpu_util import check_all, oracle_for, run_gpu, say
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

THREADS = 16


_CACHE = {}


def inputs_and_oracle(name):
    """Inputs and fp64 oracle results of a workload, computed once per session."""
    if name not in _CACHE:
        wl = get_workload(name)
        t0 = time.time()
        say(f"case {name}: generating inputs")
        inp = make_inputs(wl, threads=THREADS)
        say(f"case {name}: running the oracle ({time.time() - t0:.1f}s)")
        ref = oracle_for(wl, inp, threads=THREADS)
        _CACHE.clear()  # keep one workload's arrays at a time
        _CACHE[name] = (wl, inp, ref)
    return _CACHE[name]


@pytest.mark.parametrize("path", ["auto", "given_lse"])
@pytest.mark.parametrize("name", ["llama8b_32k_tsp", "batched_8x32k_ar1", "qwen7b_512k", "structkv_128k_16l"])
def test_full_workload(path, name):
    wl, inp, ref = inputs_and_oracle(name)
    t0 = time.time()
    say(f"case {name} [{path}]: running the HIP path")
    if path == "given_lse":
        # kvsel_score_lse with the oracle's exact LSE rounded to fp32: the
        # oracle's scores are the reference (they were computed with that LSE)
        gpu = run_gpu(wl, inp, lse_in=ref["lse"].astype(np.float32))
    else:
        gpu = run_gpu(wl, inp, path=path)
    say(f"case {name} [{path}]: comparing ({time.time() - t0:.1f}s)")
    check_all(wl, inp, gpu, ref)
    say(f"case {name} [{path}]: done ({time.time() - t0:.1f}s)")
