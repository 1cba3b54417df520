"""The four bf16 workloads at their full sizes, in the launch configuration
the benchmark times (one scoring call over every layer), against the fp64
oracle on every score, LSE, kept index and gathered row."""

import time

import pytest

from gpu_util import check_all, oracle_for, run_gpu, say
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

THREADS = 16


@pytest.mark.parametrize("name", ["llama8b_32k_tsp", "batched_8x32k_ar1", "qwen7b_512k", "structkv_128k_16l"])
def test_full_workload(name):
    wl = get_workload(name)
    t0 = time.time()
    say(f"case {name}: generating inputs")
    inp = make_inputs(wl, threads=THREADS)
    say(f"case {name}: running the HIP path ({time.time() - t0:.1f}s)")
    gpu = run_gpu(wl, inp)
    say(f"case {name}: running the oracle ({time.time() - t0:.1f}s)")
    ref = oracle_for(wl, inp, threads=THREADS)
    say(f"case {name}: comparing ({time.time() - t0:.1f}s)")
    check_all(wl, inp, gpu, ref)
    say(f"case {name}: done ({time.time() - t0:.1f}s)")
