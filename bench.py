"""Benchmark: attention-saliency token selection on one MI355X.

One step is the whole path over one batch of seeded synthetic input resident
in HBM: score every key of every layer (one kvsel_score call that also sums
the layers), select per KV head (kvsel_topk), gather the kept K and V rows of
every layer (two kvsel_gather calls). The default workload is the 128K-token
StructKV-style configuration: 16 layers of 32 query / 8 KV heads x 128,
N = 131072, w = 32, pool 7, 4096 kept per KV head.

Prints one JSON line (rank 0). ``value`` is keys scored+selected per second
(layer x sequence x KV head x key units per second of step time).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
PROFILES = os.path.join(ROOT, "profiles")
# sources of the kernels one kvsel_score call launches on the bf16 path
SCORE_SOURCES = ("token_selection_amd/csrc/stream.hip+token_selection_amd/csrc/score.hip"
                 "+token_selection_amd/csrc/tile32.h")
# ... and with the pivot statistics, also the per-layer summary kernel
STATS_SOURCES = SCORE_SOURCES + "+token_selection_amd/csrc/pivot.hip"
# decode attention; one CentroidKV round (its ranking runs the top-k kernels)
DECODE_SOURCES = "token_selection_amd/csrc/decode.hip"
CSM_SOURCES = "token_selection_amd/csrc/centroid.hip+token_selection_amd/csrc/topk.hip"


def recorded_traffic(kernel: str, sources: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3 PMC
    summaries under profiles/, if they were taken on the current sources of
    that kernel (the sha256 of the '+'-joined files, read in order, matches)
    and on the same workload; otherwise None."""
    import hashlib
    import re

    if not os.path.isdir(PROFILES):
        return None
    h = hashlib.sha256()
    for src in sources.split("+"):
        path = os.path.join(ROOT, src)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    sha = h.hexdigest()
    pat = re.compile(r"traffic: kernel=(\S+) workload=(\S+) source=(\S+) sha256=([0-9a-f]+) bytes_per_launch=(\d+)")
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        for m in pat.finditer(open(os.path.join(PROFILES, name)).read()):
            if m.group(1) == kernel and m.group(2) == workload and m.group(3) == sources and m.group(4) == sha:
                return int(m.group(5))
    return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, inp, budget_s: float = 15.0, mode: str = "two-pass", lse=None, small_p=None,
                 pool_type: str = "avg") -> dict:
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: the first n layers of every sequence and KV head through
    score -> accumulate -> select -> gather (with the LSE handed in, or plus
    the row statistics, as the timed mode does), n chosen for ~budget_s
    seconds."""
    import oracle

    cores = _cores()

    def run(n):
        t0 = time.perf_counter()
        oracle.pipeline(inp["q"][:n], inp["k"][:n], inp["v"][:n], dtype=wl.dtype, window=wl.window,
                        pool_kernel=wl.pool_kernel, kv_budget=wl.kv_budget, threads=cores,
                        lse_in=None if lse is None else lse[:n], pool_type=pool_type)
        if mode == "stats":
            oracle.row_stats_all(inp["q"][:n], inp["k"][:n], wl.dtype, small_p, threads=cores)
        return time.perf_counter() - t0

    t1 = run(1)
    n = 1
    if t1 < budget_s / 2 and wl.n_layers > 1:
        n = int(max(1, min(wl.n_layers, round(budget_s / t1))))
        t = run(n)
    else:
        t = t1
    units = n * wl.batch * wl.n_kv_heads * wl.n_keys
    return {"value": units / t, "unit": "keys/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {wl.n_layers} layers x {wl.batch} seq x {wl.n_kv_heads} KV heads x {wl.n_keys} keys "
                      f"(score{' from the given LSE' if lse is not None else ''}{', max pool' if pool_type == 'max' else ''}, "
                      f"layer sum, select, K/V gather"
                      f"{', row statistics' if mode == 'stats' else ''}) in {t:.1f} s on {cores} threads"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="structkv_128k_16l")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lse-in", action="store_true",
                    help="score with the window rows' LSE handed in (kvsel_score_lse, one pass over K); the LSE "
                         "is computed once before timing, as prefill attention would have it")
    ap.add_argument("--stats", action="store_true",
                    help="score with the pivot statistics of every window row (kvsel_score_stats, then "
                         "kvsel_layer_summary), as StructKV's pivot detection runs it")
    ap.add_argument("--max-pool", action="store_true",
                    help="pool each layer's raw scores with the max pool (then sum the layers) instead of the "
                         "average pool")
    ap.add_argument("--decode", action="store_true",
                    help="time one decode step of attention over the 16-layer 128K workload's compacted cache "
                         "(kvsel_decode_attention) instead of the selection path")
    ap.add_argument("--csm", action="store_true",
                    help="time one CentroidKV chunked-soft-matching round (kvsel_csm) on the batched 8 x 32K "
                         "workload instead of the selection path")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch every kernel from Python each step instead of replaying HIP graphs")
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto",
                    help="read 1 GiB before every timed step (auto: when the step's inputs are below 1 GiB, so "
                         "that they cannot sit in the 256 MB memory-side cache from the previous step)")
    ap.add_argument("--serial", dest="concurrent", action="store_false",
                    help="run every call on one stream (default: the token-set head mean and top-k beside the "
                         "per-head top-k, on a second stream)")
    ap.add_argument("--check", action="store_true",
                    help="after timing, compare every output of the timed step (graph replay or launches) with a "
                         "serial eager step, bit for bit; exit 1 on a difference")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer 3 times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.stats and args.lse_in:
        print("--stats and --lse-in are separate modes", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}))
        return 0

    from token_selection_amd import kvsel as K
    from workloads import get_workload, make_inputs

    if args.decode or args.csm:
        return bench_extra(args, K, get_workload, make_inputs)

    wl = get_workload(args.workload)
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = make_inputs(wl, threads=_cores())
    print(f"[bench] inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def up(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k, v = up(inp["q"]), up(inp["k"]), up(inp["v"])
    hidden = None
    if wl.tsp_budget is not None and inp.get("hidden") is not None:
        hidden = torch.from_numpy(inp["hidden"].view(np.int16)).to(dev).view(torch.bfloat16).unsqueeze(1)
    B, Hkv, N, w = wl.batch, wl.n_kv_heads, wl.n_keys, wl.window
    scores = torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, wl.kv_budget), dtype=torch.int32, device=dev)
    pool_type = K.KVSEL_POOL_MAX if args.max_pool else K.KVSEL_POOL_AVG
    desc = K.score_desc(q, k, w, wl.pool_kernel, 0.0, pool_type)
    ws = torch.empty(max(1, K.kvsel_score_workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    kc = torch.empty((wl.n_layers, B, Hkv, wl.kv_budget, wl.head_dim), dtype=k.dtype, device=dev)
    vc = torch.empty_like(kc)
    tsp = None
    if wl.tsp_budget is not None:
        tsp = {"score": torch.empty((B, 1, N - w), dtype=torch.float32, device=dev),
               "idx": torch.empty((B, 1, wl.tsp_budget), dtype=torch.int32, device=dev)}
        if hidden is not None:
            tsp["hidden"] = torch.empty((B, 1, wl.tsp_budget, hidden.shape[-1]), dtype=hidden.dtype, device=dev)
    tk_ws = torch.empty(max(1, K.kvsel_topk_workspace_bytes(B, Hkv, N, w, wl.kv_budget)), dtype=torch.uint8,
                        device=dev)
    tsp_ws = None if tsp is None else torch.empty(
        max(1, K.kvsel_topk_workspace_bytes(B, 1, N, w, wl.tsp_budget)), dtype=torch.uint8, device=dev)

    lse_in = None
    if args.lse_in:
        lse_in = torch.empty(tuple(q.shape[:4]), dtype=torch.float32, device=dev)
        K.kvsel_score(q, k, scores, window=w, pool_kernel=wl.pool_kernel, workspace=ws, desc=desc, lse_out=lse_in)
        torch.cuda.synchronize()
    small_p = 1.0 / N  # keys below the uniform share
    stats = None
    if args.stats:
        L, Hq = wl.n_layers, wl.n_q_heads
        stats = {"entropy": torch.empty((L, B, Hq, w), dtype=torch.float32, device=dev),
                 "sum_p2": torch.empty((L, B, Hq, w), dtype=torch.float32, device=dev),
                 "n_below": torch.empty((L, B, Hq, w), dtype=torch.int32, device=dev),
                 "summary": torch.empty((L, 3), dtype=torch.float32, device=dev)}

    # the stages of one step; every buffer is allocated above, so a stage is
    # kernel launches only and can be captured in a HIP graph
    def stage_score():
        if stats is not None:
            K.kvsel_score_stats(q, k, scores, window=w, pool_kernel=wl.pool_kernel, small_p=small_p, workspace=ws,
                                desc=desc, out=(stats["entropy"], stats["sum_p2"], stats["n_below"]))
            K.kvsel_layer_summary(stats["entropy"], stats["sum_p2"], stats["n_below"], n_keys=N,
                                  out=stats["summary"])
        elif lse_in is None:
            K.kvsel_score(q, k, scores, window=w, pool_kernel=wl.pool_kernel, workspace=ws, desc=desc)
        else:
            K.kvsel_score_lse(q, k, lse_in, scores, window=w, pool_kernel=wl.pool_kernel, workspace=ws, desc=desc)

    # The token-set chain (head mean, then its top-k: seven small launches)
    # runs beside the per-head top-k on a second stream (same priority),
    # joining back before the stage returns, so the stages stay in order;
    # graph capture records the fork and join as dependencies. The gathers
    # stay on one stream: each streams at full HBM rate, and a fork and join
    # in the graph costs about 10 us (measured: gather stage 0.039 against
    # 0.028 ms on the 32K workload).
    aux = torch.cuda.Stream(dev)
    mode = {"concurrent": args.concurrent}

    def side_by_side(main_fn, side_fns):
        if not mode["concurrent"] or not side_fns:
            main_fn()
            for f in side_fns:
                f()
            return
        cur = torch.cuda.current_stream(dev)
        aux.wait_stream(cur)
        with torch.cuda.stream(aux):
            for f in side_fns:
                f()
        main_fn()
        cur.wait_stream(aux)

    def tsp_chain():
        K.kvsel_accumulate(scores, tsp["score"], mode=K.KVSEL_ACC_HEAD_MEAN)
        K.kvsel_topk(tsp["score"], n_keys=N, window=w, budget=wl.tsp_budget, idx=tsp["idx"], workspace=tsp_ws)

    def stage_topk():
        side_by_side(lambda: K.kvsel_topk(scores, n_keys=N, window=w, budget=wl.kv_budget, idx=idx, workspace=tk_ws),
                     [tsp_chain] if tsp is not None else [])

    def stage_gather():
        K.kvsel_gather(k, idx, kc)
        K.kvsel_gather(v, idx, vc)
        if tsp is not None and "hidden" in tsp:
            K.kvsel_gather(hidden, tsp["idx"], tsp["hidden"])

    stages = {"score": stage_score, "topk": stage_topk, "gather": stage_gather}

    def step():
        for fn in stages.values():
            fn()

    def outputs():
        out = {"scores": scores, "idx": idx, "kc": kc, "vc": vc}
        if tsp is not None:
            out.update({"tsp_" + n: t for n, t in tsp.items()})
        if stats is not None:
            out.update({"stats_" + n: t for n, t in stats.items()})
        return out

    stream = torch.cuda.current_stream(dev)
    step()  # the library's one-time set-up (device attributes, scratch lookups) happens outside any capture
    torch.cuda.synchronize()
    # one HIP graph per stage and one for the whole step (kernel nodes only:
    # the library launches no memset or copy)
    graphs = {}
    if args.graph:
        side = torch.cuda.Stream(dev)
        for name, fn in list(stages.items()) + [("step", step)]:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                fn()
            graphs[name] = g
        torch.cuda.synchronize()
        for g in graphs.values():  # the first replay of a graph also uploads it: keep that out of the timing
            g.replay()
        torch.cuda.synchronize()
    launch = {name: (graphs[name].replay if args.graph else fn) for name, fn in list(stages.items()) + [("step", step)]}

    flusher = cache_flusher(dev, wl.compulsory_bytes()["k_read"], args.flush)
    flush = flusher is not None

    # the warm-up steps, in the timed launch form and right before the timed
    # region: the part lowers its clocks while idle (as during the graph
    # capture above) and takes about ten steps of this load to raise them
    for _ in range(args.warmup):
        if flusher is not None:
            flusher()
        launch["step"]()

    def mk():
        return torch.cuda.Event(enable_timing=True)

    def timed_runs(fn, reps):
        """reps runs of fn, each between two events on the launch stream."""
        evs = [(mk(), mk()) for _ in range(reps)]
        for e0, e1 in evs:
            if flusher is not None:
                flusher()
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    # timed region: exactly `steps` steps, synchronised on both sides
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    step_ms = timed_runs(launch["step"], args.steps)
    wall = time.perf_counter() - t_wall
    # the stages timed on their own (same launch form), for the stage split
    # and the roofline of the scoring call
    stage_runs = {name: timed_runs(launch[name], args.steps) for name in stages}

    def med(x):
        y = sorted(x)
        return y[len(y) // 2] if len(y) % 2 else 0.5 * (y[len(y) // 2 - 1] + y[len(y) // 2])

    ms_per_step = sum(step_ms) / len(step_ms)
    stage_ms = {n: med(x) for n, x in stage_runs.items()}

    check = None
    if args.check:
        # the buffers now hold the last timed stage runs' results (score, top-k, gather in order); one
        # serial eager step must reproduce every byte
        got = {n: t.clone() for n, t in outputs().items()}
        mode["concurrent"] = False
        step()
        torch.cuda.synchronize()
        bad = [n for n, t in outputs().items()
               if not torch.equal(t.contiguous().view(torch.uint8), got[n].contiguous().view(torch.uint8))]
        check = "identical" if not bad else "differs: " + ", ".join(bad)

    cb = wl.compulsory_bytes()
    units = wl.units
    value = units / (ms_per_step / 1e3)
    score_alg_bytes = cb["k_read"] + cb["q_read"] + wl.batch * wl.n_kv_heads * wl.n_prefix * 4
    achieved = score_alg_bytes / (stage_ms["score"] / 1e3) / 1e9
    whole_gbs = cb["total"] / (ms_per_step / 1e3) / 1e9
    kernel_name = ("kvsel_score_stats" if args.stats else "kvsel_score" if lse_in is None else "kvsel_score_lse")
    if args.max_pool:
        kernel_name += "_maxpool"  # its own profile: the max pool reads every layer's raw scores
    traffic = recorded_traffic(kernel_name, STATS_SOURCES if args.stats else SCORE_SOURCES, wl.name)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, mode="stats" if args.stats else "lse-in" if lse_in is not None else "two-pass",
                           lse=None if lse_in is None else lse_in.cpu().numpy().astype(np.float64),
                           small_p=small_p, pool_type="max" if args.max_pool else "avg")
        cpu["cpu_model"] = cpu_model()

    line = {
        "metric": "keys scored+selected/sec and achieved HBM GB/s (% of peak), 128K ctx",
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": med(step_ms),
        "ms_per_step_min": min(step_ms),
        "ms_per_step_max": max(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "batch": wl.batch, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "n_keys": wl.n_keys, "window": wl.window,
                   "pool": wl.pool_kernel, "pool_type": "max" if args.max_pool else "avg",
                   "kv_budget": wl.kv_budget, "tsp_budget": wl.tsp_budget,
                   "lse": "computed (two passes)" if lse_in is None else "handed in (one pass)",
                   "pivot_stats": bool(args.stats), "launch": "hip graph" if args.graph else "eager",
                   "token_set_chain": ("beside the per-head top-k" if args.concurrent else "after it")
                   if wl.tsp_budget is not None else None,
                   "cache_flush_between_steps": bool(flush)},
        "hbm_gbs_whole_path": whole_gbs,
        "hbm_frac_whole_path": whole_gbs / HBM_PEAK_GBS,
        "stage_ms": stage_ms,
        # dominant launch group: the scoring call, timed with HIP events on its
        # launch stream (median of `steps` runs); algorithmic bytes = K read
        # once + Q + final scores
        "roofline": {"bound": "hbm",
                     "kernel": ("kvsel_score_stats (stream_kernel pass 1 + merge + pass 2 + count + pool + "
                                "layer summary)" if args.stats else
                                "kvsel_score (stream_kernel pass 1 + merge + pass 2 + pool)" if lse_in is None
                                else "kvsel_score_lse (stream_kernel pass 2 + pool)")
                     + (", max pool" if args.max_pool else ""),
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "traffic_gbs": None if traffic is None else traffic / (stage_ms["score"] / 1e3) / 1e9,
                     "algorithmic_bytes": score_alg_bytes},
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }
    if check is not None:
        line["check"] = check
    print(json.dumps(line))
    return 0 if check in (None, "identical") else 1


def cache_flusher(dev, footprint_bytes: int, mode: str):
    """Cache hygiene between timed calls: with mode "on", or "auto" and inputs
    below 1 GiB (they could sit in the 256 MB memory-side cache from the
    previous call), a function that reads a 1 GiB buffer; None otherwise. It
    runs before a call's start event, outside the timing. A read, not a
    write: a written buffer leaves that cache full of dirty lines, and the
    timed call's first kernel would pay their write-back (on the batched
    8 x 32K workload: pass 1 in 157 instead of 113 us)."""
    import torch

    if not (mode == "on" or (mode == "auto" and footprint_bytes < (1 << 30))):
        return None
    buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    return lambda: buf.sum()


def timed(fn, stream, steps, warmup, flusher=None):
    """Warm-up calls, then `steps` calls, each between two HIP events on the
    launch stream (after `flusher`, if given): (mean, median, min, max) ms
    per call."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        if flusher is not None:
            flusher()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    med = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
    return sum(t) / len(t), med, t[0], t[-1]


def bench_extra(args, K, get_workload, make_inputs) -> int:
    """The two steps beside the selection path: decode attention over the
    compacted cache, and one CentroidKV clustering round."""
    import numpy as np
    import torch

    import_oracle = not args.no_cpu_baseline
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    if args.decode:
        wl = get_workload("structkv_128k_16l")
        inp = make_inputs(wl, threads=_cores())
        q, k, v = up(inp["q"]), up(inp["k"]), up(inp["v"])
        L, B, Hq, Hkv, N, w, d, bud = (wl.n_layers, wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_keys, wl.window,
                                       wl.head_dim, wl.kv_budget)
        scores = K.kvsel_score(q, k, window=w, pool_kernel=wl.pool_kernel)
        idx = K.kvsel_topk(scores, n_keys=N, window=w, budget=bud)
        kc = K.kvsel_gather(k, idx).view(L * B, Hkv, bud, d)
        vc = K.kvsel_gather(v, idx).view(L * B, Hkv, bud, d)
        qd = q[:, :, :, w - 1].contiguous().view(L * B, Hq, d)  # the newest query of every head and layer
        del k, v, q, scores
        out = torch.empty((L * B, Hq, d), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, K.kvsel_decode_workspace_bytes(L * B, Hq, Hkv, d, bud)), dtype=torch.uint8,
                         device=dev)
        flusher = cache_flusher(dev, kc.numel() * 2 + vc.numel() * 2, args.flush)
        ms, ms_med, ms_min, ms_max = timed(lambda: K.kvsel_decode_attention(qd, kc, vc, out=out, workspace=ws),
                                           stream, args.steps, args.warmup, flusher)
        units = L * B * Hkv * bud
        alg = 2 * units * d * 2 + L * B * Hq * d * (2 + 4)
        cpu = None
        if import_oracle:
            import oracle

            kh = kc.view(torch.int16).cpu().numpy().view(np.uint16)
            vh = vc.view(torch.int16).cpu().numpy().view(np.uint16)
            qh = qd.view(torch.int16).cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            n = 0
            for r in range(L * B):
                oracle.decode_attention(oracle.to_f64(qh[r], "bf16"), oracle.to_f64(kh[r], "bf16"),
                                        oracle.to_f64(vh[r], "bf16"), None, 1.0 / d ** 0.5)
                n += 1
                if time.perf_counter() - t0 > 15.0:
                    break
            t = time.perf_counter() - t0
            cpu = {"value": n * Hkv * bud / t, "unit": "keys/s", "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
                   "sample": f"{n} of {L * B} (layer, sequence) decode steps over {Hkv} KV heads x {bud} kept keys "
                             f"in {t:.1f} s"}
        line = {"metric": "decode attention over the compacted cache: kept keys attended/sec", "value": units / ms * 1e3,
                "unit": "keys/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
                "ms_per_step_median": ms_med, "ms_per_step_min": ms_min, "ms_per_step_max": ms_max,
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded; no dataset or weights)",
                "config": {"workload": "structkv_128k_16l compacted (4096 kept per KV head, 16 layers)",
                           "decode_batch": L * B, "q_heads": Hq, "kv_heads": Hkv, "keys": bud, "head_dim": d,
                           "cache_flush_between_steps": flusher is not None},
                "roofline": {"bound": "hbm", "kernel": "kvsel_decode_attention (decode_kernel + combine)",
                             "achieved": alg / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": recorded_traffic("kvsel_decode_attention", DECODE_SOURCES,
                                                         "structkv_128k_16l_compacted"),
                             "algorithmic_bytes": alg},
                "cpu_baseline": cpu}
        print(json.dumps(line))
        return 0

    wl = get_workload("batched_8x32k_ar1")
    inp = make_inputs(wl, with_hidden=False, threads=_cores())
    k, v = up(inp["k"]), up(inp["v"])
    S = wl.n_layers * wl.batch * wl.n_kv_heads
    n, d, chunk, ns, nr, rate = wl.n_keys, wl.head_dim, 64, 4, 32, 0.25
    nm = K.csm_merge_count(rate, n, ns, nr)
    flusher = cache_flusher(dev, k.numel() * 2 + v.numel() * 2, args.flush)
    ms, ms_med, ms_min, ms_max = timed(lambda: K.kvsel_csm(k, v, chunk=chunk, n_sink=ns, n_recent=nr, n_merge=nm),
                                       stream, args.steps, args.warmup, flusher)
    n_out = n - nm
    alg = 2 * S * n * d * 2 + 2 * S * n_out * d * 2 + S * n_out * 4
    cpu = None
    if import_oracle:
        import oracle

        kh = inp["k"].reshape(S, n, d)
        vh = inp["v"].reshape(S, n, d)
        t0 = time.perf_counter()
        oracle.csm_round(oracle.to_f64(kh[0], "bf16"), oracle.to_f64(vh[0], "bf16"), None, chunk, ns, nr, nm)
        t = time.perf_counter() - t0
        cpu = {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"1 of {S} slabs ({n} tokens, one CSM round) in {t:.1f} s"}
    line = {"metric": "CentroidKV chunked soft matching: cache tokens clustered/sec", "value": S * n / ms * 1e3,
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "ms_per_step_median": ms_med, "ms_per_step_min": ms_min, "ms_per_step_max": ms_max,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; no dataset or weights)",
            "config": {"workload": "batched_8x32k_ar1 keys and values", "slabs": S, "tokens": n, "head_dim": d,
                       "chunk": chunk, "n_sink": ns, "n_recent": nr, "rate": rate, "n_merge": nm,
                       "cache_flush_between_steps": flusher is not None},
            "roofline": {"bound": "hbm", "kernel": "kvsel_csm (match + select + merge)",
                         "achieved": alg / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("kvsel_csm", CSM_SOURCES, wl.name), "algorithmic_bytes": alg},
            "cpu_baseline": cpu}
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
