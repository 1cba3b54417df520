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


def recorded_traffic(kernel: str, sources: str):
    """HBM bytes per launch of `kernel` from the rocprofv3 PMC summaries under
    profiles/, if they were taken on the current sources of that kernel (the
    sha256 of the '+'-joined files, read in order, matches); otherwise None."""
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
    pat = re.compile(r"traffic: kernel=(\S+) source=(\S+) sha256=([0-9a-f]+) bytes_per_launch=(\d+)")
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        for m in pat.finditer(open(os.path.join(PROFILES, name)).read()):
            if m.group(1) == kernel and m.group(2) == sources and m.group(3) == sha:
                return int(m.group(4))
    return None


def _cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, inp, budget_s: float = 15.0, mode: str = "two-pass", lse=None, small_p=None) -> dict:
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
                        lse_in=None if lse is None else lse[:n])
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
                      f"(score{' from the given LSE' if lse is not None else ''}, layer sum, select, K/V gather"
                      f"{', row statistics' if mode == 'stats' else ''}) in {t:.1f} s on {cores} threads"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="structkv_128k_16l")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lse-in", action="store_true",
                    help="score with the window rows' LSE handed in (kvsel_score_lse, one pass over K); the LSE "
                         "is computed once before timing, as prefill attention would have it")
    ap.add_argument("--stats", action="store_true",
                    help="score with the pivot statistics of every window row (kvsel_score_stats, then "
                         "kvsel_layer_summary), as StructKV's pivot detection runs it")
    ap.add_argument("--decode", action="store_true",
                    help="time one decode step of attention over the 16-layer 128K workload's compacted cache "
                         "(kvsel_decode_attention) instead of the selection path")
    ap.add_argument("--csm", action="store_true",
                    help="time one CentroidKV chunked-soft-matching round (kvsel_csm) on the batched 8 x 32K "
                         "workload instead of the selection path")
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
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v = up(inp["q"]), up(inp["k"]), up(inp["v"])
    B, Hkv, N, w = wl.batch, wl.n_kv_heads, wl.n_keys, wl.window
    scores = torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, wl.kv_budget), dtype=torch.int32, device=dev)
    desc = K.score_desc(q, k, w, wl.pool_kernel)
    ws = torch.empty(max(1, K.kvsel_score_workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    kc = torch.empty((wl.n_layers, B, Hkv, wl.kv_budget, wl.head_dim), dtype=k.dtype, device=dev)
    vc = torch.empty_like(kc)
    stream = torch.cuda.current_stream(dev)

    stages = ("score", "topk", "gather")

    def mk():
        return torch.cuda.Event(enable_timing=True)

    lse_in = None
    if args.lse_in:
        lse_in = torch.empty(tuple(q.shape[:4]), dtype=torch.float32, device=dev)
        K.kvsel_score(q, k, scores, window=w, pool_kernel=wl.pool_kernel, workspace=ws, desc=desc, lse_out=lse_in)
        torch.cuda.synchronize()

    small_p = 1.0 / N  # keys below the uniform share

    def step(evs=None):
        # evs: per-stage (start, end) events recorded on the launch stream
        if evs:
            evs["score"][0].record(stream)
        if args.stats:
            _, ent, sp2, nb = K.kvsel_score_stats(q, k, scores, window=w, pool_kernel=wl.pool_kernel,
                                                  small_p=small_p, workspace=ws, desc=desc)
            K.kvsel_layer_summary(ent, sp2, nb, n_keys=N)
        elif lse_in is None:
            K.kvsel_score(q, k, scores, window=w, pool_kernel=wl.pool_kernel, workspace=ws, desc=desc)
        else:
            K.kvsel_score_lse(q, k, lse_in, scores, window=w, pool_kernel=wl.pool_kernel, workspace=ws, desc=desc)
        if evs:
            evs["score"][1].record(stream)
            evs["topk"][0].record(stream)
        K.kvsel_topk(scores, n_keys=N, window=w, budget=wl.kv_budget, idx=idx)
        if evs:
            evs["topk"][1].record(stream)
            evs["gather"][0].record(stream)
        K.kvsel_gather(k, idx, kc)
        K.kvsel_gather(v, idx, vc)
        if evs:
            evs["gather"][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps back to back, one event pair around all of them
    # and one around each stage of each step, all on the launch stream
    per_step = [{n: (mk(), mk()) for n in stages} for _ in range(args.steps)]
    t_begin, t_end = mk(), mk()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    t_begin.record(stream)
    for i in range(args.steps):
        step(per_step[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = t_begin.elapsed_time(t_end) / args.steps
    stage_ms = {n: sum(e[n][0].elapsed_time(e[n][1]) for e in per_step) / args.steps for n in stages}

    cb = wl.compulsory_bytes()
    units = wl.units
    value = units / (ms_per_step / 1e3)
    score_alg_bytes = cb["k_read"] + cb["q_read"] + wl.batch * wl.n_kv_heads * wl.n_prefix * 4
    achieved = score_alg_bytes / (stage_ms["score"] / 1e3) / 1e9
    whole_gbs = cb["total"] / (ms_per_step / 1e3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, mode="stats" if args.stats else "lse-in" if lse_in is not None else "two-pass",
                           lse=None if lse_in is None else lse_in.cpu().numpy().astype(np.float64),
                           small_p=small_p)

    line = {
        "metric": "keys scored+selected/sec and achieved HBM GB/s (% of peak), 128K ctx",
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "batch": wl.batch, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "n_keys": wl.n_keys, "window": wl.window,
                   "pool": wl.pool_kernel, "kv_budget": wl.kv_budget,
                   "lse": "computed (two passes)" if lse_in is None else "handed in (one pass)",
                   "pivot_stats": bool(args.stats)},
        "hbm_gbs_whole_path": whole_gbs,
        "hbm_frac_whole_path": whole_gbs / HBM_PEAK_GBS,
        "stage_ms": stage_ms,
        # dominant launch group: the scoring call (kvsel_score: stream_kernel
        # pass 1, the LSE merge, stream_kernel pass 2 and the pool, 89% of the
        # step's kernel time; with --lse-in kvsel_score_lse: the LSE copy,
        # pass 2 and the pool), timed with HIP events on its launch stream;
        # algorithmic bytes = K read once + Q + final scores
        "roofline": {"bound": "hbm",
                     "kernel": ("kvsel_score_stats (stream_kernel pass 1 + merge + pass 2 + count + pool + "
                                "layer summary)" if args.stats else
                                "kvsel_score (stream_kernel pass 1 + merge + pass 2 + pool)" if lse_in is None
                                else "kvsel_score_lse (stream_kernel pass 2 + pool)"),
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (recorded_traffic("kvsel_score_stats", STATS_SOURCES) if args.stats else
                                 recorded_traffic("kvsel_score" if lse_in is None else "kvsel_score_lse",
                                                  SCORE_SOURCES)),
                     "algorithmic_bytes": score_alg_bytes},
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }
    print(json.dumps(line))
    return 0


def timed(fn, stream, steps, warmup):
    """Warm-up calls, then `steps` calls between two HIP events on the launch
    stream: mean ms per call."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


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
        ms = timed(lambda: K.kvsel_decode_attention(qd, kc, vc, out=out, workspace=ws), stream, args.steps,
                   args.warmup)
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
            cpu = {"value": n * Hkv * bud / t, "unit": "keys/s", "cores": 1, "kind": "oracle",
                   "sample": f"{n} of {L * B} (layer, sequence) decode steps over {Hkv} KV heads x {bud} kept keys "
                             f"in {t:.1f} s"}
        line = {"metric": "decode attention over the compacted cache: kept keys attended/sec", "value": units / ms * 1e3,
                "unit": "keys/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded; no dataset or weights)",
                "config": {"workload": "structkv_128k_16l compacted (4096 kept per KV head, 16 layers)",
                           "decode_batch": L * B, "q_heads": Hq, "kv_heads": Hkv, "keys": bud, "head_dim": d},
                "roofline": {"bound": "hbm", "kernel": "kvsel_decode_attention (decode_kernel + combine)",
                             "achieved": alg / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": recorded_traffic("kvsel_decode_attention", DECODE_SOURCES),
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
    ms = timed(lambda: K.kvsel_csm(k, v, chunk=chunk, n_sink=ns, n_recent=nr, n_merge=nm), stream, args.steps,
               args.warmup)
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
        cpu = {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"1 of {S} slabs ({n} tokens, one CSM round) in {t:.1f} s"}
    line = {"metric": "CentroidKV chunked soft matching: cache tokens clustered/sec", "value": S * n / ms * 1e3,
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; no dataset or weights)",
            "config": {"workload": "batched_8x32k_ar1 keys and values", "slabs": S, "tokens": n, "head_dim": d,
                       "chunk": chunk, "n_sink": ns, "n_recent": nr, "rate": rate, "n_merge": nm},
            "roofline": {"bound": "hbm", "kernel": "kvsel_csm (match + select + merge)",
                         "achieved": alg / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("kvsel_csm", CSM_SOURCES), "algorithmic_bytes": alg},
            "cpu_baseline": cpu}
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
