"""Seeded random shapes through the streaming path, checked against the fp64
oracle to the same bar as the other parity tests (scores, LSE, kept indices,
gathered rows). The draws cover what the fixed cases only sample: the
segment cut of each slab (one or more segments per work-group slot, ragged
last chunks), head groups past 256 window rows, group sizes 1-8, both head
dims, windows from 1 to 80 and budgets from the window alone to every key."""

import numpy as np
import pytest

from gpu_util import check_all, oracle_for, run_gpu, say
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

TINY = get_workload("tiny_f32_2k")


def draw(i):
    rng = np.random.default_rng(7000 + i)
    L = int(rng.integers(1, 3))
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.integers(1, 9))
    d = int(rng.choice([64, 128]))
    w = int(rng.choice([1, 3, 8, 16, 32, 40, 64, 80]))
    N = int(rng.integers(w, 3000))
    pool = int(rng.choice([1, 3, 5, 7]))
    budget = int(rng.integers(w, N + 1))
    return L, B, G * Hkv, Hkv, d, N, w, pool, budget


CASES = [draw(i) for i in range(24)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_random_shape(case):
    L, B, Hq, Hkv, d, N, w, pool, budget = case
    say("case random", case)
    wl = TINY.with_(name="random", wid=700 + CASES.index(case), dtype="bf16", n_layers=L, batch=B, n_q_heads=Hq,
                    n_kv_heads=Hkv, head_dim=d, n_keys=N, window=w, pool_kernel=pool, kv_budget=budget,
                    n_hubs=min(8, max(0, N - w - 1)))
    inp = make_inputs(wl)
    gpu = run_gpu(wl, inp)
    ref = oracle_for(wl, inp)
    check_all(wl, inp, gpu, ref)
