"""kvsel_score_stats (StructKV section 2 pivot statistics) against the fp64
oracle: each window row's entropy, sum of p^2 and count of keys below the
threshold, the per-layer summary, and the pivot found on layers whose
attention is planted to turn sharp at a known layer.

Tolerances: entropy |gpu - oracle| <= 1e-4 + 2e-5 * (|LSE| + 1) (it is the
difference of two fp32 terms of the LSE's size); sum p^2 relative 1e-3 (as
the scores); the count may differ from the oracle's only by keys whose log
probability lies within 1e-4 + 2e-5 * (|LSE| + |logit|) of ln(small_p) (the
GPU decides on fp32 logits)."""

import math
import time

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_lse_close, assert_scores_close, oracle_for, say, to_dev
from token_selection_amd import kvsel as K
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

TINY = get_workload("tiny_f32_2k")


def run_stats(wl, inp, small_p):
    q = to_dev(inp["q"], wl.dtype)
    k = to_dev(inp["k"], wl.dtype)
    L, B, Hq, w, _ = inp["q"].shape
    lse = torch.full((L, B, Hq, w), float("nan"), device=q.device)
    scores, ent, sp2, nb = K.kvsel_score_stats(q, k, window=wl.window, pool_kernel=wl.pool_kernel, small_p=small_p,
                                               lse_out=lse)
    summary = K.kvsel_layer_summary(ent, sp2, nb, n_keys=wl.n_keys)
    torch.cuda.synchronize()
    out = {"scores": scores.cpu().numpy(), "lse": lse.cpu().numpy(), "entropy": ent.cpu().numpy(),
           "sum_p2": sp2.cpu().numpy(), "n_below": nb.cpu().numpy(), "summary": summary.cpu().numpy()}
    del q, k
    return out


def near_threshold(wl, inp, small_p, l, b, h):
    """Per window row of (layer l, sequence b, head h): the oracle's count of
    visible keys whose log probability is within the decision band of ln(small_p)."""
    d = wl.head_dim
    G = wl.group
    qh = oracle.to_f64(inp["q"][l, b, h], wl.dtype)
    kg = oracle.to_f64(inp["k"][l, b, h // G], wl.dtype)
    logits = oracle.window_logits(qh, kg, oracle.default_scale(d))
    lse = oracle.row_lse(logits)
    vis = np.isfinite(logits)
    lp = np.where(vis, logits - lse[:, None], 0.0)
    band = 1e-4 + 2e-5 * (np.abs(lse)[:, None] + np.abs(np.where(vis, logits, 0.0)))
    return (vis & (np.abs(lp - math.log(small_p)) <= band)).sum(axis=1)


def check_stats(wl, inp, gpu, small_p, heads=None, ref_stats=None):
    ent, sp2, nb = ref_stats if ref_stats is not None else oracle.row_stats_all(
        inp["q"], inp["k"], wl.dtype, small_p, threads=8)
    L, B, Hq, w = ent.shape
    hs = range(Hq) if heads is None else heads
    ref = oracle_for(wl, inp) if ref_stats is None else None
    lse_ref = ref["lse"] if ref is not None else None
    for l in range(L):
        for b in range(B):
            for h in hs:
                lse = lse_ref[l, b, h] if lse_ref is not None else gpu["lse"][l, b, h].astype(np.float64)
                tol = 1e-4 + 2e-5 * (np.abs(lse) + 1.0)
                err = np.abs(gpu["entropy"][l, b, h] - ent[l, b, h])
                assert (err <= tol).all(), f"entropy (l={l}, b={b}, h={h}): max err {err.max()} " \
                                           f"gpu {gpu['entropy'][l, b, h][:4]} oracle {ent[l, b, h][:4]}"
                e2 = np.abs(gpu["sum_p2"][l, b, h] - sp2[l, b, h])
                assert (e2 <= 1e-3 * sp2[l, b, h] + 1e-30).all(), f"sum_p2 (l={l}, b={b}, h={h}): {e2.max()}"
                dn = np.abs(gpu["n_below"][l, b, h].astype(np.int64) - nb[l, b, h])
                if dn.any():
                    near = near_threshold(wl, inp, small_p, l, b, h)
                    assert (dn <= near).all(), f"n_below (l={l}, b={b}, h={h}): off by {dn.max()}, band {near.max()}"
    return ref


# (L, B, Hq, Hkv, d, N, w, pool) -- bf16
SHAPES = [
    (1, 1, 4, 1, 128, 3001, 5, 7),      # ragged last chunk, G = 4
    (2, 2, 6, 2, 64, 2500, 7, 3),       # d = 64, G = 3, 2 layers, 2 sequences
    (1, 1, 28, 4, 128, 4100, 16, 7),    # 112 rows
    (1, 1, 8, 8, 128, 1111, 1, 1),      # w = 1
    (1, 1, 8, 2, 128, 777, 64, 5),      # 256 rows
    (1, 2, 4, 2, 128, 40, 40, 7),       # w = N: no prefix, only window keys
    (1, 1, 4, 2, 128, 41, 40, 7),       # one prefix key
    (2, 1, 28, 4, 64, 2100, 64, 7),     # 448 rows: head groups of 4 and 3 heads, 2 layers
    (5, 4, 8, 8, 128, 25076, 16, 7),    # 5 layers, 4 sequences, 8 KV heads, 25K keys
]


@pytest.mark.parametrize("small_p", [1e-4, 3e-3])
@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "-".join(map(str, c)))
def test_row_stats(case, small_p):
    L, B, Hq, Hkv, d, N, w, pool = case
    say("case stats", case, small_p)
    wl = TINY.with_(name="stats", wid=500 + SHAPES.index(case), dtype="bf16", n_layers=L, batch=B, n_q_heads=Hq,
                    n_kv_heads=Hkv, head_dim=d, n_keys=N, window=w, pool_kernel=pool, kv_budget=w,
                    n_hubs=min(8, max(0, N - w - 1)))
    inp = make_inputs(wl, with_v=False)
    gpu = run_stats(wl, inp, small_p)
    ref = check_stats(wl, inp, gpu, small_p)
    # the scores and LSE of the same call are kvsel_score's
    assert_scores_close(gpu["scores"], ref["scores"])
    assert_lse_close(gpu["lse"], ref["lse"])
    # the summary kernel: the oracle's summary of the GPU's own row statistics
    me, ms, mv = oracle.layer_summary(gpu["entropy"].astype(np.float64), gpu["sum_p2"].astype(np.float64),
                                      gpu["n_below"], N)
    np.testing.assert_allclose(gpu["summary"][:, 0], me, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(gpu["summary"][:, 1], ms, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(gpu["summary"][:, 2], mv, rtol=1e-5, atol=1e-12)


def test_large_logits_stats():
    """Keys x 100 (logits of several hundred): the overflow guard of the
    statistics' fast path must send blocks to the row-maximum path."""
    wl = TINY.with_(name="stats_big", wid=520, dtype="bf16", head_dim=128, k_mult=100.0, n_keys=3000, window=16,
                    kv_budget=16, n_hubs=0, hub_mode=None)
    say("case stats large logits")
    inp = make_inputs(wl, with_v=False)
    gpu = run_stats(wl, inp, 1e-3)
    check_stats(wl, inp, gpu, 1e-3)


def test_uniform_rows_closed_form():
    """q = 0: every row is uniform, so entropy = ln n_i, sum p^2 = 1/n_i and the
    count is n_i or 0 on either side of 1/n_i (closed forms, no oracle run)."""
    N, w = 5000, 24
    wl = TINY.with_(name="stats_zero", wid=521, dtype="bf16", head_dim=128, query_model="zero", n_keys=N, window=w,
                    kv_budget=w, n_hubs=0, hub_mode=None)
    say("case stats uniform")
    inp = make_inputs(wl, with_v=False)
    n = N - w + 1 + np.arange(w)
    for small_p, full in ((1.0 / (N - w + 1) * 1.01, True), (1.0 / N * 0.99, False)):
        gpu = run_stats(wl, inp, small_p)
        np.testing.assert_allclose(gpu["entropy"], np.broadcast_to(np.log(n), gpu["entropy"].shape), rtol=2e-6)
        np.testing.assert_allclose(gpu["sum_p2"], np.broadcast_to(1.0 / n, gpu["sum_p2"].shape), rtol=1e-4)
        assert (gpu["n_below"] == (n if full else 0)).all()


def test_planted_pivot():
    """Layers 0-3 with unit keys, layers 4-7 with keys x 3: the attention turns
    sharp at layer 4 (entropy falls by about half, sparsity rises). The GPU's
    summary gives pivot 4 through kvsel_pivot_layer, as does the oracle's."""
    mult = (1.0, 1.05, 0.95, 1.0, 3.0, 3.1, 2.9, 3.0)
    wl = TINY.with_(name="pivot", wid=530, dtype="bf16", n_layers=8, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    n_keys=4000, window=16, kv_budget=16, n_hubs=0, hub_mode=None, layer_k_mult=mult)
    small_p = 1.0 / 4000
    say("case planted pivot")
    inp = make_inputs(wl, with_v=False)
    gpu = run_stats(wl, inp, small_p)
    ref_stats = oracle.row_stats_all(inp["q"], inp["k"], "bf16", small_p, threads=8)
    check_stats(wl, inp, gpu, small_p, ref_stats=ref_stats)
    me, ms, _ = oracle.layer_summary(*ref_stats, wl.n_keys)
    assert oracle.pivot_layer(me, ms, 0.2, 0.1) == 4
    summ = gpu["summary"]
    assert K.kvsel_pivot_layer(summ[:, 0], summ[:, 1], min_drop=0.2, min_rise=0.1) == 4
    np.testing.assert_allclose(summ[:, 0], me, rtol=1e-4)
    np.testing.assert_allclose(summ[:, 1], ms, atol=2e-3)


def test_stats_unsupported_shape_raises():
    """fp32 (the general path) has no statistics: the call fails loudly."""
    wl = TINY
    inp = make_inputs(wl, with_v=False)
    q = to_dev(inp["q"], "f32")
    k = to_dev(inp["k"], "f32")
    with pytest.raises(K.KvselError):
        K.kvsel_score_stats(q, k, window=wl.window, small_p=1e-3)


@pytest.mark.parametrize("name", ["llama8b_32k_tsp", "structkv_128k_16l"])
def test_full_size_sampled_heads(name):
    """Full-size workloads in the benchmark's launch configuration, checked on
    sampled query heads (the oracle computes one head at a time)."""
    wl = get_workload(name)
    t0 = time.time()
    say(f"case stats {name}: inputs")
    inp = make_inputs(wl, with_v=False, with_hidden=False, threads=16)
    small_p = 1.0 / wl.n_keys
    say(f"case stats {name}: HIP ({time.time() - t0:.1f}s)")
    gpu = run_stats(wl, inp, small_p)
    L, B, Hq, w, d = inp["q"].shape
    rng = np.random.default_rng(77)
    picks = [(int(rng.integers(L)), int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(6)]
    say(f"case stats {name}: oracle on {picks} ({time.time() - t0:.1f}s)")
    for (l, b, h) in picks:
        g = h // wl.group
        qh = oracle.to_f64(inp["q"][l, b, h:h + 1], wl.dtype)
        kg = oracle.to_f64(inp["k"][l, b, g:g + 1], wl.dtype)
        ent, sp2, nb = oracle.row_stats(qh, kg, small_p)
        lse = oracle.row_lse(oracle.window_logits(qh[0], kg[0], oracle.default_scale(d)))
        tol = 1e-4 + 2e-5 * (np.abs(lse) + 1.0)
        assert (np.abs(gpu["entropy"][l, b, h] - ent[0]) <= tol).all()
        assert (np.abs(gpu["sum_p2"][l, b, h] - sp2[0]) <= 1e-3 * sp2[0]).all()
        dn = np.abs(gpu["n_below"][l, b, h].astype(np.int64) - nb[0])
        if dn.any():
            assert (dn <= near_threshold(wl, inp, small_p, l, b, h)).all()
    # the call's scores are kvsel_score's (checked against the oracle at full size elsewhere), up to
    # the rounding of the two calls' LSE merges
    q = to_dev(inp["q"], wl.dtype)
    k = to_dev(inp["k"], wl.dtype)
    plain = K.kvsel_score(q, k, window=wl.window, pool_kernel=wl.pool_kernel).cpu().numpy()
    np.testing.assert_allclose(gpu["scores"].astype(np.float64), plain.astype(np.float64), rtol=1e-5, atol=1e-30)
    say(f"case stats {name}: done ({time.time() - t0:.1f}s)")
