"""HIP path vs the fp64 oracle, element by element, on seeded inputs at sizes
the oracle finishes in seconds: the tiny fp32 workload in full, ragged and
degenerate shapes that span several tiles, accumulation, the token-set path,
exact ties, large logits, determinism and output coverage."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_gather, assert_scores_close, assert_selection, check_all, device, oracle_for,
                      run_gpu, say, stream_eligible, to_dev)
from token_selection_amd import kvsel as K
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

TINY = get_workload("tiny_f32_2k")


def test_tiny_workload_full():
    say("case tiny_f32_2k full")
    inp = make_inputs(TINY)
    gpu = run_gpu(TINY, inp)
    ref = oracle_for(TINY, inp)
    check_all(TINY, inp, gpu, ref)
    # behaviour (not parity): the 16 planted hubs are kept in both heads
    hubs = inp["hub_pos"]
    for g in range(TINY.n_kv_heads):
        assert set(hubs) <= set(gpu["idx"][0, g].tolist())


# (dtype, L, B, Hq, Hkv, d, N, w, pool, budget)
RAGGED = [
    ("bf16", 1, 1, 4, 1, 128, 3001, 5, 7, 300),     # ragged last chunk, G=4, w=5 -> 20 rows
    ("bf16", 2, 2, 6, 2, 64, 2500, 7, 3, 999),      # G=3, 21 rows, 2 layers
    ("bf16", 1, 1, 28, 4, 128, 4100, 16, 7, 512),   # G=7 -> 112 rows (7 row blocks)
    ("bf16", 1, 1, 14, 1, 128, 1500, 20, 7, 100),   # 280 rows: streamed as 2 head groups of 7 heads
    ("bf16", 1, 1, 8, 8, 128, 1111, 1, 1, 1),       # w=1, budget=w, G=1
    ("bf16", 1, 1, 8, 2, 128, 777, 64, 5, 777),     # budget = N
    ("bf16", 1, 2, 4, 2, 128, 40, 40, 7, 40),       # w = N: empty prefix
    ("bf16", 1, 1, 4, 2, 128, 41, 40, 7, 41),       # one prefix key
    ("f32", 1, 1, 8, 2, 64, 2049, 32, 7, 256),      # fp32, ragged
    ("f32", 3, 1, 4, 2, 128, 1300, 9, 3, 60),       # fp32 d=128, 3 layers
    ("f32", 1, 1, 12, 4, 64, 5000, 33, 1, 4000),    # fp32, pool 1, large budget
    ("bf16", 1, 1, 64, 8, 128, 2048, 128, 7, 1024), # 1024 rows: 4 head groups of 2 heads
    ("bf16", 2, 1, 28, 4, 64, 3333, 64, 7, 400),    # G=7, w=64 (448 rows): groups of 4 and 3 heads, 2 layers
]


def _skip_if_not_streamable(wl, path):
    if path == "stream" and not stream_eligible(wl):
        pytest.skip("the streaming kernels do not take this shape (the explicit choice returns UNSUPPORTED, "
                    "checked in test_stream_path_refuses_other_shapes)")


@pytest.mark.parametrize("path", ["auto", "stream", "general"])
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "-".join(map(str, c)))
def test_ragged_shapes(case, path):
    """Every scoring path the library has, chosen explicitly through the
    descriptor (the library's report of the kernels it runs is checked)."""
    dt, L, B, Hq, Hkv, d, N, w, pool, budget = case
    say("case ragged", case, path)
    wl = TINY.with_(name="ragged", wid=100 + RAGGED.index(case), dtype=dt, n_layers=L, batch=B, n_q_heads=Hq,
                    n_kv_heads=Hkv, head_dim=d, n_keys=N, window=w, pool_kernel=pool, kv_budget=budget,
                    n_hubs=min(8, max(0, N - w - 1)))
    _skip_if_not_streamable(wl, path)
    inp = make_inputs(wl)
    gpu = run_gpu(wl, inp, path=path)
    ref = oracle_for(wl, inp)
    check_all(wl, inp, gpu, ref)


def layer_groups(L, B, Hq, Hkv, d, N, w):
    """Layers per group of the streamed pass 2's layer sums for this shape
    (average pool, one head group), or 0 where every layer keeps its own raw
    row: as many layers per group as leave each of the 2 x n_CU work-group
    slots a unit of 8192 keys of one (b, KV head)."""
    n_wg = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    R = Hq // Hkv * w
    rbn = 1
    while rbn * 32 < R:
        rbn *= 2
    Np = N - w
    if L < 2 or Np <= 0 or R > 256 or not ((d == 128 and rbn <= 4) or (d == 64 and rbn <= 8)):
        return 0
    per_group = B * Hkv * -(-Np // 8192)
    n_groups = -(-n_wg // per_group)
    return 0 if n_groups >= L else -(-L // n_groups)


# (L, B, Hq, Hkv, d, N, w, pool, budget, KV heads checked, layers per group on 256 CUs)
LAYER_SUM = [
    (16, 1, 32, 8, 128, 5 * 8192 + 140, 32, 7, 2048, (0, 5), 2),  # 128 rows, 8 groups of 2 layers
    (5, 4, 8, 8, 128, 3 * 8192 + 500, 16, 7, 1000, (3,), 2),      # groups of 2, 2 and 1 layers, 4 sequences
    (3, 2, 128, 16, 64, 60000, 32, 5, 3000, (1, 14), 2),          # d = 64, 256 rows, groups of 2 and 1
    (3, 4, 16, 16, 64, 4 * 8192 + 1008, 8, 7, 900, (7,), 2),      # 640 units on 512 work-groups
]


@pytest.mark.parametrize("case", LAYER_SUM, ids=lambda c: "-".join(map(str, c[:9])))
def test_layer_sum_pass2(case):
    """Calls whose pass 2 sums groups of layers in LDS (long prefixes, many
    layers, average pool): every score and LSE of the checked KV heads against
    the oracle's, the call added to earlier scores (accumulate), and the
    single-pass call given the two-pass call's own LSE, which must reproduce
    its scores up to that LSE's rounding."""
    L, B, Hq, Hkv, d, N, w, pool, budget, hs, lg = case
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    if n_cu == 256:  # the premise: this shape takes the layer-sum pass
        assert layer_groups(L, B, Hq, Hkv, d, N, w) == lg
    say("case layer sum", case, "layers per group", layer_groups(L, B, Hq, Hkv, d, N, w))
    wl = TINY.with_(name="layer_sum", wid=540 + LAYER_SUM.index(case), dtype="bf16", n_layers=L, batch=B,
                    n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_keys=N, window=w, pool_kernel=pool,
                    kv_budget=budget, n_hubs=16)
    inp = make_inputs(wl, threads=16, with_v=False)
    ref = oracle_for(wl, inp, heads=hs)
    gpu = run_gpu(wl, inp, with_gather=False)
    check_all(wl, inp, gpu, ref, heads=hs)
    prev = np.random.default_rng(5).uniform(0.0, 2.0, size=gpu["scores"].shape).astype(np.float32)
    acc = run_gpu(wl, inp, accumulate_into=prev, with_gather=False, with_lse=False)
    assert_scores_close(acc["scores"][:, list(hs)], prev[:, list(hs)] + ref["scores"][:, list(hs)])
    one = run_gpu(wl, inp, lse_in=gpu["lse"], with_gather=False)
    np.testing.assert_allclose(one["scores"].astype(np.float64), gpu["scores"].astype(np.float64), rtol=1e-5,
                               atol=1e-30)


def test_stream_path_refuses_other_shapes():
    """An explicit streaming choice on fp32 input is refused before any
    launch, with UNSUPPORTED, and nothing is written."""
    wl = TINY
    inp = make_inputs(wl)
    q, k = to_dev(inp["q"], "f32"), to_dev(inp["k"], "f32")
    scores = torch.full((1, wl.n_kv_heads, wl.n_keys - wl.window), 7.0, device=device())
    desc = K.score_desc(q, k, wl.window, wl.pool_kernel, path=K.KVSEL_PATH_STREAM)
    assert K.kvsel_score_path(desc) == -1
    with pytest.raises(K.KvselError) as e:
        K.kvsel_score(q, k, scores, window=wl.window, desc=desc)
    assert e.value.status == K.KVSEL_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((scores == 7.0).all())


MAXPOOL_CASES = [RAGGED[0], RAGGED[1], RAGGED[6], RAGGED[7], RAGGED[9], RAGGED[10], RAGGED[3], RAGGED[12]]


@pytest.mark.parametrize("path", ["auto", "general"])
@pytest.mark.parametrize("case", MAXPOOL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_max_pool(case, path):
    """The max-pool variant on every scoring path: per-layer max over the pool
    window, then the layer sum (multi-layer cases check that order)."""
    dt, L, B, Hq, Hkv, d, N, w, pool, budget = case
    say("case max-pool", case, path)
    wl = TINY.with_(name="maxpool", wid=400 + MAXPOOL_CASES.index(case), dtype=dt, n_layers=L, batch=B,
                    n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_keys=N, window=w, pool_kernel=pool,
                    kv_budget=budget, n_hubs=min(8, max(0, N - w - 1)))
    inp = make_inputs(wl)
    gpu = run_gpu(wl, inp, pool_type=K.KVSEL_POOL_MAX, path=path)
    ref = oracle_for(wl, inp, pool_type=K.KVSEL_POOL_MAX)
    check_all(wl, inp, gpu, ref)


def test_max_pool_given_lse():
    """Max pool through the single-pass entry point."""
    wl = TINY.with_(name="maxpool_lse", wid=420, dtype="bf16", head_dim=128, n_layers=2, n_keys=3000, window=16,
                    kv_budget=300)
    say("case max-pool given lse")
    inp = make_inputs(wl)
    lse = oracle_for(wl, inp)["lse"].astype(np.float32)
    gpu = run_gpu(wl, inp, lse_in=lse, pool_type=K.KVSEL_POOL_MAX)
    ref = oracle_for(wl, inp, lse_in=lse.astype(np.float64), pool_type=K.KVSEL_POOL_MAX)
    check_all(wl, inp, gpu, ref)


@pytest.mark.parametrize("n_sink", [1, 4, 37, "all"])
def test_sinks_are_kept(n_sink):
    """kvsel_topk_sinks: the first n_sink positions are always kept and the
    rest of the budget is the top of the other prefix positions, in both the
    per-KV-head and the token-set selections; "all" fills the whole non-window
    budget with sinks."""
    wl = get_workload("llama8b_32k_tsp").with_(name="sinks", wid=430, n_keys=5000, n_hubs=50, hidden_dim=136,
                                               kv_budget=200, tsp_budget=400)
    ns = wl.kv_budget - wl.window if n_sink == "all" else n_sink
    say("case sinks", ns)
    inp = make_inputs(wl)
    gpu = run_gpu(wl, inp, n_sink=ns)
    ref = oracle_for(wl, inp, n_sink=ns)
    check_all(wl, inp, gpu, ref, n_sink=ns)


def test_sinks_with_low_scores():
    """Sinks whose scores are the lowest of the row (planted through the
    scores buffer directly) still come first; ties among the others go to the
    lower position."""
    B, H, N, w, budget, ns = 2, 3, 4000, 8, 100, 10
    rng = np.random.default_rng(431)
    sc = rng.random((B, H, N - w)).astype(np.float32) + 1.0
    sc[..., :ns] = 0.0
    sc[..., 500:700] = 2.5  # a tie block larger than the budget
    say("case sinks low scores")
    idx = K.kvsel_topk(torch.from_numpy(sc).to(device()), n_keys=N, window=w, budget=budget, n_sink=ns)
    got = idx.cpu().numpy()
    exp = list(range(ns)) + list(range(500, 500 + budget - w - ns)) + list(range(N - w, N))
    for b in range(B):
        for h in range(H):
            assert got[b, h].tolist() == exp
            assert got[b, h].tolist() == oracle.select_row(sc[b, h].astype(np.float64), N, w, budget, ns).tolist()


def test_rope_sink_tsp_small():
    """The token-set (TSP) path on a reduced 32K-style layer: RoPE, a sink,
    hubs, head mean, one token set per sequence, hidden-row gather."""
    wl = get_workload("llama8b_32k_tsp").with_(n_keys=6000, n_hubs=60, hidden_dim=136, batch=2,
                                               kv_budget=300, tsp_budget=700)
    say("case tsp small")
    inp = make_inputs(wl)
    gpu = run_gpu(wl, inp)
    ref = oracle_for(wl, inp)
    check_all(wl, inp, gpu, ref)
    assert 0 in gpu["tsp_idx"][0, 0]  # the sink survives


def test_accumulate_flag_adds_layers():
    """scores(accumulate) = previous content + this call's layer sum; two
    calls of 2 layers equal one call of 4 layers (StructKV accumulation)."""
    wl = TINY.with_(name="acc", wid=140, dtype="bf16", head_dim=128, n_layers=4, n_keys=3000, window=16,
                    kv_budget=400, hub_mode="norm", hub_scale=3.0, hub_layers=1, n_hubs=20)
    say("case accumulate")
    inp = make_inputs(wl)
    ref = oracle_for(wl, inp)
    q = to_dev(inp["q"], "bf16")
    k = to_dev(inp["k"], "bf16")
    s1 = K.kvsel_score(q[:2], k[:2], window=wl.window, pool_kernel=7)
    K.kvsel_score(q[2:], k[2:], s1, window=wl.window, pool_kernel=7, accumulate=True)
    s4 = K.kvsel_score(q, k, window=wl.window, pool_kernel=7)
    torch.cuda.synchronize()
    assert_scores_close(s1.cpu().numpy(), ref["scores"])
    assert_scores_close(s4.cpu().numpy(), ref["scores"])
    # one layer at a time through kvsel_accumulate(ADD)
    acc = torch.zeros_like(s4)
    for l in range(4):
        sl = K.kvsel_score(q[l], k[l], window=wl.window, pool_kernel=7)
        K.kvsel_accumulate(sl, acc, K.KVSEL_ACC_ADD)
    torch.cuda.synchronize()
    assert_scores_close(acc.cpu().numpy(), ref["scores"])


@pytest.mark.parametrize("pool_type", [K.KVSEL_POOL_AVG, K.KVSEL_POOL_MAX])
def test_accumulate_with_head_groups(pool_type):
    """Accumulation across calls with 448 window rows per KV head (G = 7,
    w = 64: two head groups): two calls of 2 layers equal one call of 4 layers
    and the oracle's layer sum, with either pool."""
    wl = TINY.with_(name="acc_hg", wid=145, dtype="bf16", head_dim=128, n_layers=4, n_q_heads=28, n_kv_heads=4,
                    n_keys=1500, window=64, kv_budget=300, n_hubs=20)
    say("case accumulate head groups", pool_type)
    inp = make_inputs(wl)
    ref = oracle_for(wl, inp, pool_type=pool_type)
    q = to_dev(inp["q"], "bf16")
    k = to_dev(inp["k"], "bf16")
    s1 = K.kvsel_score(q[:2], k[:2], window=wl.window, pool_kernel=7, pool_type=pool_type)
    K.kvsel_score(q[2:], k[2:], s1, window=wl.window, pool_kernel=7, pool_type=pool_type, accumulate=True)
    s4 = K.kvsel_score(q, k, window=wl.window, pool_kernel=7, pool_type=pool_type)
    torch.cuda.synchronize()
    assert_scores_close(s1.cpu().numpy(), ref["scores"])
    assert_scores_close(s4.cpu().numpy(), ref["scores"])


def test_exact_ties_follow_tie_break():
    """q = 0 makes every prefix score bit-identical on the GPU too; the
    tie-break alone decides: pool 1 keeps [0, kk), pool 7 keeps [3, kk + 3)."""
    for pool, first in ((1, 0), (7, 3)):
        wl = TINY.with_(name="ties", wid=150, dtype="bf16", head_dim=128, query_model="zero", n_keys=5000,
                        window=24, pool_kernel=pool, kv_budget=1000, n_hubs=0, hub_mode=None)
        say("case ties pool", pool)
        inp = make_inputs(wl)
        gpu = run_gpu(wl, inp, with_gather=False)
        kk = wl.kv_budget - wl.window
        exp = list(range(first, first + kk)) + list(range(wl.n_prefix, wl.n_keys))
        for g in range(wl.n_kv_heads):
            assert gpu["idx"][0, g].tolist() == exp
            interior = gpu["scores"][0, g, 3:-3]
            assert np.all(interior == interior[0])
        ref = oracle_for(wl, inp)
        assert_scores_close(gpu["scores"], ref["scores"])


@pytest.mark.parametrize("path", ["auto", "general"])
@pytest.mark.parametrize("k_mult,lse_floor", [(100.0, 300.0), (300.0, 900.0)])
def test_large_logits_are_stable(k_mult, lse_floor, path):
    """Keys x 100 push logits to several hundred, keys x 300 to about +-1000:
    the two-pass softmax must subtract row maxima (fp32 exp overflows past
    88), so the first-logit reference of pass 1 falls back to the row maximum
    and every LSE still matches the oracle's."""
    wl = TINY.with_(name="big", wid=160, dtype="bf16", head_dim=128, k_mult=k_mult, n_keys=3000, window=16,
                    kv_budget=200, n_hubs=0, hub_mode=None)
    say("case large logits", k_mult, path)
    inp = make_inputs(wl)
    ref = oracle_for(wl, inp)
    assert np.abs(ref["lse"]).max() > lse_floor  # the premise: logits of the stated size
    gpu = run_gpu(wl, inp, path=path)
    check_all(wl, inp, gpu, ref)


def test_deterministic_and_fully_written():
    """Two runs give bit-identical scores and indices; outputs pre-filled with
    NaN / -1 are fully overwritten and guard bands around them stay intact."""
    wl = get_workload("llama8b_32k_tsp").with_(n_keys=9000, n_hubs=90, tsp_budget=None, hidden_dim=None,
                                               kv_budget=700)
    say("case determinism")
    inp = make_inputs(wl, with_v=False)
    q = to_dev(inp["q"], "bf16")
    k = to_dev(inp["k"], "bf16")
    B, H, Np = 1, wl.n_kv_heads, wl.n_prefix
    guard = 4096
    runs = []
    for rep in range(2):
        sbuf = torch.full((B * H * Np + 2 * guard,), float("nan"), device=device())
        ibuf = torch.full((B * H * wl.kv_budget + 2 * guard,), -7, dtype=torch.int32, device=device())
        scores = sbuf[guard:guard + B * H * Np].view(B, H, Np)
        idx = ibuf[guard:guard + B * H * wl.kv_budget].view(B, H, wl.kv_budget)
        K.kvsel_score(q, k, scores, window=wl.window, pool_kernel=7)
        K.kvsel_topk(scores, n_keys=wl.n_keys, window=wl.window, budget=wl.kv_budget, idx=idx)
        torch.cuda.synchronize()
        sb, ib = sbuf.cpu().numpy(), ibuf.cpu().numpy()
        assert np.isnan(sb[:guard]).all() and np.isnan(sb[-guard:]).all()
        assert (ib[:guard] == -7).all() and (ib[-guard:] == -7).all()
        assert np.isfinite(sb[guard:-guard]).all()
        assert (ib[guard:-guard] >= 0).all()
        runs.append((sb[guard:-guard].copy(), ib[guard:-guard].copy()))
    assert runs[0][0].tobytes() == runs[1][0].tobytes()
    assert np.array_equal(runs[0][1], runs[1][1])


def test_strided_query_view():
    """q_win may be a strided view of a larger query tensor (only the last w
    positions of every head)."""
    wl = TINY.with_(name="strided", wid=170, dtype="bf16", head_dim=128, n_keys=2500, window=12, kv_budget=100)
    say("case strided q")
    inp = make_inputs(wl, with_v=False)
    L, B, Hq, w, d = inp["q"].shape
    big = np.zeros((L, B, Hq, 50, d), dtype=np.uint16)
    big[:, :, :, 50 - w:] = inp["q"]
    qbig = to_dev(big, "bf16")
    k = to_dev(inp["k"], "bf16")
    s = K.kvsel_score(qbig[:, :, :, 50 - w:], k, window=w, pool_kernel=7)
    torch.cuda.synchronize()
    ref = oracle_for(wl, inp)
    assert_scores_close(s.cpu().numpy(), ref["scores"])


LSE_CASES = [c for c in RAGGED if c[0] == "bf16"] + [RAGGED[8], RAGGED[9]]


@pytest.mark.parametrize("path", ["auto", "general"])
@pytest.mark.parametrize("case", LSE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_scores_from_given_lse(case, path):
    """kvsel_score_lse (single pass, the window rows' LSE handed in) against the
    oracle given the same LSE: the true LSE (fp32-rounded) and one shifted per
    row by seeded offsets, so that the result is not the self-normalised one."""
    dt, L, B, Hq, Hkv, d, N, w, pool, budget = case
    say("case given-lse", case, path)
    wl = TINY.with_(name="given_lse", wid=300 + LSE_CASES.index(case), dtype=dt, n_layers=L, batch=B,
                    n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_keys=N, window=w, pool_kernel=pool,
                    kv_budget=budget, n_hubs=min(8, max(0, N - w - 1)))
    inp = make_inputs(wl)
    ref0 = oracle_for(wl, inp)
    offs = np.random.default_rng(99).normal(0.0, 0.7, size=ref0["lse"].shape)
    for lse in (ref0["lse"], ref0["lse"] + offs):
        lse32 = lse.astype(np.float32)
        ref = oracle_for(wl, inp, lse_in=lse32.astype(np.float64))
        gpu = run_gpu(wl, inp, lse_in=lse32, path=path)
        check_all(wl, inp, gpu, ref)


def test_given_lse_matches_two_pass():
    """Feeding kvsel_score's own LSE back into kvsel_score_lse reproduces
    kvsel_score's scores (same data, one pass instead of two)."""
    wl = get_workload("llama8b_32k_tsp").with_(name="lse_roundtrip", wid=350, n_keys=6000, kv_budget=600,
                                               tsp_budget=900, n_hubs=60, hidden_dim=None)
    inp = make_inputs(wl)
    q = to_dev(inp["q"], wl.dtype)
    k = to_dev(inp["k"], wl.dtype)
    lse = torch.empty(inp["q"].shape[:4], dtype=torch.float32, device=device())
    s2 = K.kvsel_score(q, k, window=wl.window, pool_kernel=wl.pool_kernel, lse_out=lse)
    s1 = K.kvsel_score_lse(q, k, lse, window=wl.window, pool_kernel=wl.pool_kernel)
    a, b = s1.cpu().numpy().astype(np.float64), s2.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-30)
