"""The seeded input generators: determinism, rounding, workload readings."""

import numpy as np

from workloads import (WORKLOADS, bf16_bits_to_f32, budget_from_rate, f64_to_bf16_bits,
                       get_workload, make_inputs)
from workloads.gen import hub_positions


def test_bf16_round_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0, 0.0, 3.0e38])
    bits = f64_to_bf16_bits(x)
    assert list(bits[:5]) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000]
    back = bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[3] == -2.0


def test_rate_to_budget():
    assert budget_from_rate(0.10, 32768, 32) == 3277
    assert budget_from_rate(0.0, 100, 8) == 8
    assert budget_from_rate(1.5, 100, 8) == 100
    assert get_workload("batched_8x32k_ar1").kv_budget == 3277


def test_deterministic_and_layer_independent():
    wl = get_workload("tiny_f32_2k").with_(n_layers=3, hub_layers=2)
    a = make_inputs(wl, seed=3)
    b = make_inputs(wl, seed=3, layers=[2])
    assert np.array_equal(a["k"][2], b["k"][0]) and np.array_equal(a["q"][2], b["q"][0])
    c = make_inputs(wl, seed=4)
    assert not np.array_equal(a["k"], c["k"])


def test_workload_table_shapes():
    for wl in WORKLOADS.values():
        assert wl.n_q_heads % wl.n_kv_heads == 0
        assert wl.window <= wl.kv_budget <= wl.n_keys
        assert wl.pool_kernel % 2 == 1
    s = get_workload("structkv_128k_16l")
    assert s.units == 16 * 8 * 131072
    assert abs(s.compulsory_bytes()["total"] - 4.845e9) < 0.01e9


def test_tiny_hubs_point_along_mean_query():
    wl = get_workload("tiny_f32_2k")
    d = make_inputs(wl)
    hubs = hub_positions(wl)
    assert hubs.size == 16 and hubs.min() >= 1 and hubs.max() < wl.n_prefix
    q = d["q"][0, 0].astype(np.float64)          # [Hq, w, d]
    k = d["k"][0, 0].astype(np.float64)          # [Hkv, N, d]
    G = wl.group
    for g in range(wl.n_kv_heads):
        u = q[g * G:(g + 1) * G].reshape(-1, wl.head_dim).mean(0)
        u /= np.linalg.norm(u)
        kh = k[g, hubs]
        cos = kh @ u / np.linalg.norm(kh, axis=1)
        assert cos.min() > 0.999


def test_sink_and_ar1():
    wl = get_workload("llama8b_32k_tsp").with_(n_keys=4096, n_hubs=40, hidden_dim=64)
    d = make_inputs(wl, with_v=False)
    k = bf16_bits_to_f32(d["k"][0, 0])
    norms = np.linalg.norm(k, axis=-1)
    assert norms[:, 0].min() > 5 * np.sqrt(128) and d["hidden"].shape == (1, 4096, 64)
    wl = get_workload("batched_8x32k_ar1").with_(batch=1, n_keys=70000)
    k = bf16_bits_to_f32(make_inputs(wl, with_v=False)["k"][0, 0, 0])
    r = np.mean(np.sum(k[1:] * k[:-1], 1)) / np.mean(np.sum(k * k, 1))
    assert 0.88 < r < 0.92
    # the AR(1) state carries across independently seeded key blocks
    jump = np.linalg.norm(k[65536] - k[65535]) / np.sqrt(128)
    assert jump < 1.0
