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
