"""Helpers of the GPU parity tests: run the HIP path through the C ABI on
device copies of the seeded inputs, and compare it with the fp64 oracle.

Tolerances (the bar every GPU test applies):
* scores: |gpu - oracle| <= 1e-3 * |oracle| + 1e-30 (fp32 arithmetic; the
  floor only covers probabilities below fp32's normal range);
* LSE: |gpu - oracle| <= 1e-4 + 1e-5 * |oracle| (fp32 log2-domain maxima and
  sums; an LSE error e scales every probability of the row by exp(e));
* kept indices: the GPU's set equals the oracle's tie-broken selection applied
  to the GPU's own fp32 scores, exactly; against the oracle's fp64 scores it
  may differ only at positions whose oracle score is within 1e-3 of the
  threshold score;
* gathered rows: bit-exact.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from token_selection_amd import kvsel as K

SCORE_RTOL = 1e-3
SCORE_ATOL = 1e-30
LSE_ATOL = 1e-4
LSE_RTOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device() -> torch.device:
    if not torch.cuda.is_available():
        raise RuntimeError("this test needs a HIP device")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


PATHS = {"auto": K.KVSEL_PATH_AUTO, "stream": K.KVSEL_PATH_STREAM, "general": K.KVSEL_PATH_GENERAL}


def stream_eligible(wl) -> bool:
    """Whether the streaming kernels take this shape (what AUTO picks)."""
    return wl.dtype == "bf16" and wl.head_dim in (64, 128) and wl.window <= 256


def run_gpu(wl, inp, *, with_lse=True, with_gather=True, accumulate_into=None, lse_in=None, pool_type=0,
            n_sink=0, path="auto"):
    """The path as the benchmark runs it: one kvsel_score call over every
    layer, the per-KV-head select, the K/V gather over every layer, and (with
    a TSP budget) head mean, token-set select and hidden gather. With
    ``lse_in`` ([L, B, Hq, w] natural-log LSE) the scoring call is
    kvsel_score_lse instead. ``pool_type`` picks the pool (K.KVSEL_POOL_*),
    ``n_sink`` the protected first positions of both selections. ``path``
    ("auto", "stream", "general") picks the scoring kernels; the library's
    own report of the kernels it runs must match."""
    q = to_dev(inp["q"], wl.dtype)
    k = to_dev(inp["k"], wl.dtype)
    desc = K.score_desc(q, k, wl.window, wl.pool_kernel, 0.0, pool_type, PATHS[path])
    expect = K.KVSEL_PATH_STREAM if (path == "stream" or (path == "auto" and stream_eligible(wl))) else \
        K.KVSEL_PATH_GENERAL
    assert K.kvsel_score_path(desc) == expect, (path, K.kvsel_score_path(desc))
    L, B, Hq, w, d = inp["q"].shape
    out = {}
    lse = torch.full((L, B, Hq, w), float("nan"), device=device()) if with_lse and lse_in is None else None
    if accumulate_into is not None:
        scores = torch.from_numpy(accumulate_into.astype(np.float32)).to(device())
    else:
        scores = torch.full((B, wl.n_kv_heads, wl.n_keys - wl.window), float("nan"), device=device())
    if lse_in is None:
        K.kvsel_score(q, k, scores, window=wl.window, accumulate=accumulate_into is not None, lse_out=lse,
                      desc=desc)
    else:
        lse_dev = torch.from_numpy(np.ascontiguousarray(lse_in, dtype=np.float32)).to(device())
        K.kvsel_score_lse(q, k, lse_dev, scores, window=wl.window, accumulate=accumulate_into is not None,
                          desc=desc)
    idx = K.kvsel_topk(scores, n_keys=wl.n_keys, window=wl.window, budget=wl.kv_budget, n_sink=n_sink)
    out["scores"] = scores.cpu().numpy()
    out["idx"] = idx.cpu().numpy()
    if lse is not None:
        out["lse"] = lse.cpu().numpy()
    if with_gather and inp.get("v") is not None:
        v = to_dev(inp["v"], wl.dtype)
        out["k_kept"] = to_host(K.kvsel_gather(k, idx))
        out["v_kept"] = to_host(K.kvsel_gather(v, idx))
        del v
    if wl.tsp_budget is not None:
        tsc = K.kvsel_accumulate(scores, mode=K.KVSEL_ACC_HEAD_MEAN)
        tidx = K.kvsel_topk(tsc, n_keys=wl.n_keys, window=wl.window, budget=wl.tsp_budget, n_sink=n_sink)
        out["tsp_scores"] = tsc.cpu().numpy()
        out["tsp_idx"] = tidx.cpu().numpy()
        if inp.get("hidden") is not None:
            h = to_dev(inp["hidden"], "bf16").unsqueeze(1)  # [B, 1, N, D]
            out["hidden_kept"] = to_host(K.kvsel_gather(h, tidx))[:, 0]
            del h
    torch.cuda.synchronize()
    del q, k
    return out


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, what: str = "scores"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bad = err > SCORE_RTOL * np.abs(ref) + SCORE_ATOL
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} oracle={ref[tuple(i)]!r}")


def assert_lse_close(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = ~(err <= LSE_ATOL + LSE_RTOL * np.abs(ref))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"lse: {bad.sum()} outside tolerance; first at {tuple(i)}: gpu={gpu[tuple(i)]} "
                             f"oracle={ref[tuple(i)]}")


def assert_selection(idx_gpu: np.ndarray, scores_gpu: np.ndarray, scores_ref: np.ndarray, n_keys: int,
                     window: int, budget: int, what: str = "idx", n_sink: int = 0):
    """idx_gpu [..., budget]; scores [..., N - w]."""
    lead = idx_gpu.shape[:-1]
    ig = idx_gpu.reshape(-1, budget).astype(np.int64)
    sg = scores_gpu.reshape(ig.shape[0], n_keys - window).astype(np.float64)
    sr = scores_ref.reshape(ig.shape[0], n_keys - window)
    kk = budget - window
    for r in range(ig.shape[0]):
        row = ig[r]
        # invariants
        assert np.all(np.diff(row) > 0), f"{what}[{r}] not strictly ascending"
        assert list(row[kk:]) == list(range(n_keys - window, n_keys)), f"{what}[{r}] window not kept last"
        assert list(row[:n_sink]) == list(range(n_sink)), f"{what}[{r}] sinks not kept"
        # same decision in the same precision: oracle select on the GPU's scores
        exp_same = oracle.select_row(sg[r], n_keys, window, budget, n_sink)
        if not np.array_equal(row, exp_same):
            diff = np.setxor1d(row, exp_same)
            raise AssertionError(f"{what}[{r}] differs from the oracle's select of the GPU scores at {diff[:10]}")
        # against the oracle's own scores: only near-threshold positions may differ
        if kk > n_sink:
            exp_ref = oracle.select_row(sr[r], n_keys, window, budget, n_sink)
            diff = np.setxor1d(row[:kk], exp_ref[:kk])
            if diff.size:
                tau = np.sort(sr[r][n_sink:])[::-1][kk - n_sink - 1]
                far = diff[np.abs(sr[r][diff] - tau) > SCORE_RTOL * abs(tau) + SCORE_ATOL]
                assert far.size == 0, f"{what}[{r}] differs from the oracle away from the threshold at {far[:10]}"
    return lead


def assert_gather(kept: np.ndarray, src: np.ndarray, idx: np.ndarray, what: str):
    """kept [L, B, H, budget, d] vs src [L, B, H, N, d] at idx [B, H or 1, budget]: bit-exact."""
    L, B, H = src.shape[:3]
    for l in range(L):
        for b in range(B):
            exp = oracle.gather_rows(src[l, b], idx[b].astype(np.int64))
            if exp.tobytes() != kept[l, b].tobytes():
                raise AssertionError(f"{what}: gathered rows differ at layer {l}, batch {b}")


def oracle_for(wl, inp, threads=8, heads=None, lse_in=None, pool_type=0, n_sink=0):
    return oracle.pipeline(inp["q"], inp["k"], inp.get("v"), dtype=wl.dtype, window=wl.window,
                           pool_kernel=wl.pool_kernel, kv_budget=wl.kv_budget, tsp_budget=wl.tsp_budget,
                           hidden=inp.get("hidden"), threads=threads, heads=heads, lse_in=lse_in,
                           pool_type="max" if pool_type == K.KVSEL_POOL_MAX else "avg", n_sink=n_sink)


def check_all(wl, inp, gpu, ref, heads=None, n_sink=0):
    """Every comparison of one run (optionally restricted to some KV heads)."""
    hs = list(range(wl.n_kv_heads)) if heads is None else list(heads)
    assert_scores_close(gpu["scores"][:, hs], ref["scores"][:, hs])
    if "lse" in gpu:
        G = wl.group
        qh = [h for g in hs for h in range(g * G, (g + 1) * G)]
        assert_lse_close(gpu["lse"][:, :, qh], ref["lse"][:, :, qh])
    assert_selection(gpu["idx"][:, hs], gpu["scores"][:, hs], ref["scores"][:, hs], wl.n_keys, wl.window,
                     wl.kv_budget, n_sink=n_sink)
    if "k_kept" in gpu:
        assert_gather(gpu["k_kept"], inp["k"], gpu["idx"], "K")
        assert_gather(gpu["v_kept"], inp["v"], gpu["idx"], "V")
    if wl.tsp_budget is not None and heads is None:
        assert_scores_close(gpu["tsp_scores"], ref["tsp_scores"], "tsp_scores")
        assert_selection(gpu["tsp_idx"], gpu["tsp_scores"], ref["tsp_scores"], wl.n_keys, wl.window,
                         wl.tsp_budget, "tsp_idx", n_sink=n_sink)
        if "hidden_kept" in gpu:
            for b in range(wl.batch):
                exp = inp["hidden"][b][gpu["tsp_idx"][b, 0].astype(np.int64)]
                assert exp.tobytes() == gpu["hidden_kept"][b].tobytes(), "hidden rows differ"
