"""The selection step captured in a HIP graph (kernel nodes only: the library
launches no memset or copy) and replayed several times, with eager work of the
program in between, gives the eager step's outputs bit for bit on every replay:
scores, kept indices, gathered K/V rows, the token-set score, indices and
hidden rows."""

import numpy as np
import pytest
import torch

from gpu_util import device, say, to_dev
from token_selection_amd import kvsel as K
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    wl = get_workload("llama8b_32k_tsp").with_(name="graph", wid=470, n_layers=2, n_keys=6000, n_hubs=60,
                                               hidden_dim=136, kv_budget=300, tsp_budget=700)
    say("case graph replay", wl.name)
    inp = make_inputs(wl)
    dev = device()
    q, k, v = to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16"), to_dev(inp["v"], "bf16")
    hid = to_dev(inp["hidden"], "bf16").unsqueeze(1)
    B, Hkv, N, w = wl.batch, wl.n_kv_heads, wl.n_keys, wl.window
    desc = K.score_desc(q, k, w, wl.pool_kernel)
    ws = torch.empty(K.kvsel_score_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    tk_ws = torch.empty(max(1, K.kvsel_topk_workspace_bytes(B, Hkv, N, w, wl.kv_budget)), dtype=torch.uint8,
                        device=dev)
    ts_ws = torch.empty(max(1, K.kvsel_topk_workspace_bytes(B, 1, N, w, wl.tsp_budget)), dtype=torch.uint8,
                        device=dev)
    out = {"scores": torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev),
           "idx": torch.empty((B, Hkv, wl.kv_budget), dtype=torch.int32, device=dev),
           "kc": torch.empty((wl.n_layers, B, Hkv, wl.kv_budget, wl.head_dim), dtype=torch.bfloat16, device=dev),
           "vc": torch.empty((wl.n_layers, B, Hkv, wl.kv_budget, wl.head_dim), dtype=torch.bfloat16, device=dev),
           "tsc": torch.empty((B, 1, N - w), dtype=torch.float32, device=dev),
           "tidx": torch.empty((B, 1, wl.tsp_budget), dtype=torch.int32, device=dev),
           "hc": torch.empty((B, 1, wl.tsp_budget, hid.shape[-1]), dtype=torch.bfloat16, device=dev)}

    def step():
        K.kvsel_score(q, k, out["scores"], window=w, workspace=ws, desc=desc)
        K.kvsel_topk(out["scores"], n_keys=N, window=w, budget=wl.kv_budget, idx=out["idx"], workspace=tk_ws)
        K.kvsel_gather(k, out["idx"], out["kc"])
        K.kvsel_gather(v, out["idx"], out["vc"])
        K.kvsel_accumulate(out["scores"], out["tsc"], mode=K.KVSEL_ACC_HEAD_MEAN)
        K.kvsel_topk(out["tsc"], n_keys=N, window=w, budget=wl.tsp_budget, idx=out["tidx"], workspace=ts_ws)
        K.kvsel_gather(hid, out["tidx"], out["hc"])

    def snapshot():
        torch.cuda.synchronize()
        return {n: t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy()
                for n, t in out.items()}

    def poison():
        for t in out.values():
            t.view(torch.int32 if t.element_size() == 4 else torch.int16).fill_(-1)

    step()
    ref = snapshot()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device=dev)
    for r in range(4):
        poison()
        g.replay()
        # eager work of the program between replays (a kvsel call and torch ops)
        K.kvsel_topk(out["scores"].clone(), n_keys=N, window=w, budget=wl.kv_budget)
        other.mul_(1.0001).add_(0.5)
        got = snapshot()
        for n in ref:
            assert np.array_equal(got[n], ref[n]), f"replay {r}: {n} differs from the eager step"


def test_other_entry_points_graph_replays_match_eager():
    """The calls beside the selection step in one HIP graph: the score call
    with the pivot statistics and the per-layer summary, the single-pass call
    from a handed-in LSE, decode attention with degrees, one CSM round (its
    outputs allocated during capture) and the top-k without a workspace. Every
    replay, with the outputs poisoned before it and eager work after it,
    gives the eager results bit for bit."""
    dev = device()
    wl = get_workload("tiny_f32_2k").with_(name="graph2", wid=471, dtype="bf16", head_dim=128, n_layers=2,
                                           n_keys=3000, n_hubs=30, kv_budget=300)
    say("case graph replay (other entry points)", wl.name)
    inp = make_inputs(wl)
    q, k = to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16")
    L, B, Hq, Hkv, N, w = wl.n_layers, wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_keys, wl.window
    desc = K.score_desc(q, k, w, wl.pool_kernel)
    ws = torch.empty(K.kvsel_score_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    g = torch.Generator(device="cpu").manual_seed(471)
    lse_in = torch.empty((L, B, Hq, w), dtype=torch.float32, device=dev)
    K.kvsel_score(q, k, window=w, workspace=ws, desc=desc, lse_out=lse_in)
    qd = (torch.randn((4, 8, 128), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    kd = (torch.randn((4, 2, 1000, 128), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    vd = torch.randn((4, 2, 1000, 128), generator=g).to(torch.bfloat16).to(dev)
    deg = torch.randint(1, 5, (4, 2, 1000), generator=g, dtype=torch.int32).to(dev)
    dws = torch.empty(K.kvsel_decode_workspace_bytes(4, 8, 2, 128, 1000), dtype=torch.uint8, device=dev)
    kc = torch.randn((2, 2, 600, 64), generator=g).to(torch.bfloat16).to(dev)
    vc = torch.randn((2, 2, 600, 64), generator=g).to(torch.bfloat16).to(dev)
    ts = torch.rand((1, 3, 5000), generator=g).to(dev)
    out = {"scores": torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev),
           "entropy": torch.empty((L, B, Hq, w), dtype=torch.float32, device=dev),
           "sum_p2": torch.empty((L, B, Hq, w), dtype=torch.float32, device=dev),
           "n_below": torch.empty((L, B, Hq, w), dtype=torch.int32, device=dev),
           "summary": torch.empty((L, 3), dtype=torch.float32, device=dev),
           "scores_lse": torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev),
           "decode": torch.empty((4, 8, 128), dtype=torch.float32, device=dev),
           "idx_noalloc": torch.empty((1, 3, 300), dtype=torch.int32, device=dev)}
    csm_out = {}

    def step():
        K.kvsel_score_stats(q, k, out["scores"], window=w, small_p=1.0 / N, workspace=ws, desc=desc,
                            out=(out["entropy"], out["sum_p2"], out["n_below"]))
        K.kvsel_layer_summary(out["entropy"], out["sum_p2"], out["n_below"], n_keys=N, out=out["summary"])
        K.kvsel_score_lse(q, k, lse_in, out["scores_lse"], window=w, workspace=ws, desc=desc)
        K.kvsel_decode_attention(qd, kd, vd, deg, out=out["decode"], workspace=dws)
        kco, vco, dgo = K.kvsel_csm(kc, vc, chunk=16, n_sink=2, n_recent=8, n_merge=100)
        csm_out.update({"csm_k": kco, "csm_v": vco, "csm_deg": dgo})
        K.kvsel_topk_noalloc(ts, out["idx_noalloc"], n_keys=5000 + 8, window=8, budget=300)

    def tensors():
        return dict(out, **csm_out)

    def snapshot():
        torch.cuda.synchronize()
        return {n: t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy()
                for n, t in tensors().items()}

    step()
    ref = snapshot()
    side = torch.cuda.Stream(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device=dev)
    for r in range(4):
        for t in tensors().values():
            t.view(torch.int32 if t.element_size() == 4 else torch.int16).fill_(-1)
        graph.replay()
        K.kvsel_decode_attention(qd, kd, vd)  # eager work of the program between replays
        other.mul_(1.0001).add_(0.5)
        got = snapshot()
        for n in ref:
            assert np.array_equal(got[n], ref[n]), f"replay {r}: {n} differs from the eager call"
