"""kvsel_topk_noalloc (the top-k with its scratch in a static per-GPU array)
against kvsel_topk / kvsel_topk_sinks with a workspace, through the C ABI:
two calls in a row on the same GPU, the second smaller (and with sinks), so
the second call runs on the array the first one left behind; both must give
the workspace version's indices exactly."""

import numpy as np
import pytest
import torch

from gpu_util import device, say
from token_selection_amd import kvsel as K

pytestmark = pytest.mark.gpu


def _scores(rng, B, rows, n_prefix):
    s = rng.random((B, rows, n_prefix)).astype(np.float32)
    s[..., 100:400] = 0.75          # a block of exact ties across the threshold
    s[:, :, ::97] = 0.0
    return torch.from_numpy(s).to(device())


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_topk_matches_workspace_topk(order):
    rng = np.random.default_rng(880)
    calls = [(2, 8, 40000, 16, 1000, 0), (1, 3, 5000, 8, 300, 4)]
    for (B, rows, N, w, budget, n_sink) in calls:
        say("case topk noalloc", B, rows, N, w, budget, n_sink)
        sc = _scores(rng, B, rows, N - w)
        ref = K.kvsel_topk(sc, n_keys=N, window=w, budget=budget, n_sink=n_sink)
        got = torch.full((B, rows, budget), -7, dtype=torch.int32, device=device())
        K.kvsel_topk_noalloc(sc, got, n_keys=N, window=w, budget=budget, n_sink=n_sink)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
