"""Each kernel on its own against the oracle: top-k on crafted fp32 scores
(exact ties, many tiles, degenerate budgets), gather (vector and byte paths,
shared and per-head index sets, out-of-range indices), accumulate."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import device, say
from token_selection_amd import kvsel as K

pytestmark = pytest.mark.gpu


def _topk_case(scores_np, n_keys, window, budget):
    s = torch.from_numpy(scores_np.astype(np.float32)).to(device())
    idx = K.kvsel_topk(s, n_keys=n_keys, window=window, budget=budget)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    B, R, _ = scores_np.shape
    for b in range(B):
        for r in range(R):
            exp = oracle.select_row(scores_np[b, r].astype(np.float32).astype(np.float64), n_keys, window, budget)
            assert np.array_equal(got[b, r], exp), (b, r, np.setxor1d(got[b, r], exp)[:10])


@pytest.mark.parametrize("n_keys,window,budget,kind", [
    (100, 4, 10, "rand"), (100, 4, 4, "rand"), (100, 4, 100, "rand"), (5000, 32, 600, "ties"),
    (70000, 64, 3277, "rand"), (70000, 64, 8000, "ties"), (20000, 8, 2048, "const"), (9000, 1, 9000, "ties"),
    (131072, 32, 4096, "rand"), (4097, 1, 4096, "rand"), (300000, 64, 8192, "zeros_and_ties"),
    # around the one-launch limit of 4096 prefix keys per row (one work-group per row up to it)
    (4096 + 8, 8, 1024, "rand"), (4096 + 9, 8, 1024, "rand"), (4096 + 8, 8, 4096 + 8, "ties"),
    (4096 + 8, 8, 3000, "ties"), (33, 1, 2, "const"), (2048, 32, 256, "zeros_and_ties"), (4096 + 8, 8, 9, "const"),
    # rows of 32K keys
    (32768 + 8, 8, 2048, "rand"), (32768 + 9, 8, 2048, "rand"), (32768 + 8, 8, 32768 + 8, "ties"),
    (32768 + 8, 8, 5000, "ties"), (32768 + 8, 8, 100, "const"), (32768 + 8, 8, 4000, "zeros_and_ties"),
    # digit layouts: values over many octaves, within one ulp-scale band, of both signs
    (20000, 8, 2048, "spread"), (20000, 8, 300, "narrow"), (20000, 16, 3000, "signed"), (3000, 8, 700, "narrow"),
    (3000, 8, 500, "signed"), (4096 + 8, 8, 1500, "spread"),
    # pooled-like rows (neighbouring positions share digits), and rows of 256K keys
    (131072, 32, 4096, "smooth"), (32768 + 8, 8, 2048, "smooth"), (5000, 8, 600, "smooth"),
    (262144 + 8, 8, 5000, "rand"), (262145 + 8, 8, 5000, "ties"), (262144 + 8, 8, 3000, "smooth"),
])
def test_topk_matches_oracle(n_keys, window, budget, kind):
    say("topk", n_keys, window, budget, kind)
    rng = np.random.default_rng(n_keys + budget)
    shape = (2, 3, n_keys - window)
    if kind == "rand":
        s = rng.random(shape).astype(np.float32)
    elif kind == "ties":
        s = rng.integers(0, 7, shape).astype(np.float32) * np.float32(0.125)
    elif kind == "const":
        s = np.full(shape, 0.3, dtype=np.float32)
    elif kind == "spread":
        s = np.exp2(rng.uniform(-120.0, 120.0, shape)).astype(np.float32)
    elif kind == "narrow":
        s = (np.float32(1.0) + rng.integers(0, 40, shape).astype(np.float32) * np.float32(2.0 ** -23))
    elif kind == "signed":
        s = rng.standard_normal(shape).astype(np.float32)
    elif kind == "smooth":  # a 7-wide mean of heavy-tailed values, like pooled saliency
        raw = np.exp(rng.standard_normal(shape[:-1] + (shape[-1] + 6,)) * 2.0)
        c = np.cumsum(raw, axis=-1)
        s = ((c[..., 6:] - np.concatenate([np.zeros(shape[:-1] + (1,)), c[..., :-7]], -1)) / 7).astype(np.float32)
    else:
        s = rng.integers(0, 3, shape).astype(np.float32)
        s[..., ::5] = 0.0
    _topk_case(s, n_keys, window, budget)


@pytest.mark.parametrize("n_keys,window,budget,n_sink", [
    (3000, 8, 500, 4), (20000, 8, 2048, 16), (20000, 8, 40, 32), (20000, 8, 41, 32), (32768 + 8, 8, 4000, 1),
    (70000, 64, 3000, 7),
])
def test_topk_sinks_match_oracle(n_keys, window, budget, n_sink):
    """Protected sink positions through both kernel families (one work-group
    per row up to 4096 keys, chunked above), including sinks filling every
    slot and all slots but one."""
    say("topk sinks", n_keys, window, budget, n_sink)
    rng = np.random.default_rng(n_keys + n_sink)
    s = rng.random((2, 3, n_keys - window)).astype(np.float32)
    s[:, 1, :n_sink] = 0.0  # the sinks' own scores do not matter
    t = torch.from_numpy(s).to(device())
    idx = K.kvsel_topk(t, n_keys=n_keys, window=window, budget=budget, n_sink=n_sink)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(2):
        for r in range(3):
            exp = oracle.select_row(s[b, r].astype(np.float64), n_keys, window, budget, n_sink=n_sink)
            assert np.array_equal(got[b, r], exp), (b, r, np.setxor1d(got[b, r], exp)[:10])


def test_topk_negative_and_signed_zero():
    """The order map handles negative scores and ranks -0 equal to +0 (ties
    then go to the lower position)."""
    s = np.array([[[0.0, -0.0, 1.0, -1.0, -0.0, 0.0, 2.0, -3.0, 0.0, -0.0]]], dtype=np.float32)
    s = np.concatenate([s, s[:, :, ::-1].copy()], axis=1)
    _topk_case(s, 12, 2, 7)


# Row sizes of both 16-byte kernel forms: slab form with 4 units per item
# (64, 128, 256, 8192 bytes) or 1 (16, 32), general form (48, 192); byte copy (6, 100).
@pytest.mark.parametrize("row_bytes,idx_heads", [(256, 4), (256, 1), (128, 4), (8192, 1), (16, 4), (32, 1),
                                                 (64, 1), (48, 4), (192, 4), (6, 4), (100, 1)])
def test_gather_bit_exact(row_bytes, idx_heads):
    say("gather", row_bytes, idx_heads)
    rng = np.random.default_rng(row_bytes)
    L, B, H, N, budget = 3, 2, 4, 500, 37
    src = rng.integers(0, 256, (L, B, H, N, row_bytes), dtype=np.uint8)
    idx = np.stack([np.stack([np.sort(rng.choice(N, budget, replace=False)) for _ in range(idx_heads)])
                    for _ in range(B)]).astype(np.int32)
    out = K.kvsel_gather(torch.from_numpy(src).to(device()), torch.from_numpy(idx).to(device()))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for l in range(L):
        for b in range(B):
            exp = oracle.gather_rows(src[l, b], idx[b].astype(np.int64))
            assert exp.tobytes() == got[l, b].tobytes()


def test_gather_grid_stride():
    """More work items per slab than one grid row holds (8200 rows of 8 KB:
    1 049 600 items against 4096 work-groups of 256), so items loop."""
    say("gather grid stride")
    rng = np.random.default_rng(21)
    N, budget, row_bytes = 9000, 8200, 8192
    src = rng.integers(0, 256, (1, 1, 2, N, row_bytes), dtype=np.uint8)
    idx = np.stack([np.sort(rng.choice(N, budget, replace=False)) for _ in range(2)])[None].astype(np.int32)
    out = K.kvsel_gather(torch.from_numpy(src).to(device()), torch.from_numpy(idx).to(device()))
    torch.cuda.synchronize()
    exp = oracle.gather_rows(src[0, 0], idx[0].astype(np.int64))
    assert exp.tobytes() == out.cpu().numpy()[0, 0].tobytes()


def test_gather_strided_source_and_bad_indices():
    """A strided source (a view of every other layer) is read at its strides;
    an index outside [0, N) gives an all-zero row."""
    rng = np.random.default_rng(5)
    src = rng.integers(0, 1 << 16, (4, 1, 2, 300, 128), dtype=np.uint16)
    idx = np.array([[[0, 5, 299, 300], [-1, 7, 8, 1 << 30]]], dtype=np.int32)
    t = torch.from_numpy(src.view(np.int16)).to(device())[::2]
    out = K.kvsel_gather(t, torch.from_numpy(idx).to(device()))
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    for li, l in enumerate((0, 2)):
        for h in range(2):
            for tpos, j in enumerate(idx[0, h]):
                exp = src[l, 0, h, j] if 0 <= j < 300 else np.zeros(128, np.uint16)
                assert np.array_equal(got[li, 0, h, tpos], exp)


def test_accumulate_modes():
    rng = np.random.default_rng(8)
    src = rng.random((3, 5, 1001)).astype(np.float32)
    dst = rng.random((3, 5, 1001)).astype(np.float32)
    d = torch.from_numpy(dst).to(device())
    K.kvsel_accumulate(torch.from_numpy(src).to(device()), d, K.KVSEL_ACC_ADD)
    hm = K.kvsel_accumulate(torch.from_numpy(src).to(device()), mode=K.KVSEL_ACC_HEAD_MEAN)
    torch.cuda.synchronize()
    np.testing.assert_allclose(d.cpu().numpy(), dst.astype(np.float64) + src, rtol=1e-6)
    np.testing.assert_allclose(hm.cpu().numpy(), oracle.head_mean(src.astype(np.float64)), rtol=1e-6)
