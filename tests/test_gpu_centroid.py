"""CentroidKV chunked soft matching (kvsel_csm) and decode attention
(kvsel_decode_attention) against the fp64 oracle.

CSM decisions are floating-point choices (an argmax, a ranking), so they are
checked the way the selection is: the GPU's similarities within 2e-5 of the
oracle's cosines; each GPU match a best partner within that margin (and the
oracle's own when its best is ahead by more); the GPU's chosen set exactly the
oracle's ranking of the GPU's own fp32 similarities, and different from the
oracle's ranking of its own only at similarities within 2e-5 of the threshold.
The merge arithmetic is then checked on the GPU's decisions: survivors that
are not centroids bit for bit, centroids within one bf16 ulp of the exact
degree-weighted mean (fp32 accumulation, one rounding to bf16) plus 2^-20
times the weighted mean of the members' magnitudes (the fp32 sum's rounding
when signs cancel), degrees exactly. Decode attention: |gpu - oracle| <= 1e-4 * max|v| + 1e-4 * |oracle|
(fp32 logits of exact bf16 products, fp32 softmax)."""

import math
import time

import numpy as np
import pytest
import torch

import oracle
from gpu_util import say, to_dev, to_host
from token_selection_amd import kvsel as K
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

SIM_TOL = 2e-5
BATCHED = get_workload("batched_8x32k_ar1")


def widen(bits):
    return oracle.to_f64(bits, "bf16")


def check_csm_slab(k_bits, v_bits, deg, chunk, ns, nr, nm, gpu, s):
    """One slab: k_bits, v_bits [n, d] uint16, deg [n] int; gpu = dict of host
    arrays for this slab."""
    k = widen(k_bits)
    v = widen(v_bits)
    a_pos, score, match = oracle.csm_match(k, chunk, ns, nr)
    gs, gm, gc = gpu["score"], gpu["match"], gpu["chosen"]
    assert gs.shape == score.shape, (gs.shape, score.shape)
    fin = np.isfinite(score)
    assert (np.isfinite(gs) == fin).all(), f"slab {s}: candidates differ"
    err = np.abs(gs[fin].astype(np.float64) - score[fin])
    assert (err <= SIM_TOL).all(), f"slab {s}: similarity error {err.max()}"
    for i in np.nonzero(fin)[0]:
        a, b = int(a_pos[i]), int(gm[i])
        assert (b - a) % 2 == 1 and b > a - 64 and b < a + 64, f"slab {s}: match {b} of A {a} out of its chunk"
        cb = oracle.cosine(k[a], k[b])
        assert cb >= score[i] - SIM_TOL, f"slab {s}: A {a} matched {b} ({cb}) below best {score[i]}"
    assert (gm[~fin] == -1).all()
    # the chosen set: the oracle's ranking of the GPU's own similarities, exactly
    same = oracle.csm_select(gs.astype(np.float64), nm)
    assert np.array_equal(gc.astype(np.int64), same), f"slab {s}: chosen set differs from the ranking of GPU scores"
    own = oracle.csm_select(score, nm)
    diff = np.setxor1d(gc, own)
    if diff.size and nm > 0:
        tau = np.sort(score[fin])[::-1][nm - 1]
        far = diff[np.abs(score[diff] - tau) > SIM_TOL]
        assert far.size == 0, f"slab {s}: chosen set differs away from the threshold"
    # merge arithmetic on the GPU's decisions
    ek, ev, edeg, merged = oracle.csm_merge(k, v, deg, a_pos, gm.astype(np.int64), gc.astype(np.int64))
    # the weighted means of |x|: the scale of the fp32 sum's rounding when signs cancel
    ak, av, _, _ = oracle.csm_merge(np.abs(k), np.abs(v), deg, a_pos, gm.astype(np.int64), gc.astype(np.int64))
    assert np.array_equal(gpu["degree"].astype(np.int64), edeg), f"slab {s}: degrees differ"
    keep = np.ones(k.shape[0], dtype=bool)
    keep[a_pos[gc.astype(np.int64)]] = False
    src_rows = np.nonzero(keep)[0]
    for name, bits_in, exact, absmean in (("k", k_bits, ek, ak), ("v", v_bits, ev, av)):
        out_bits = gpu[name]
        plain = ~merged
        assert np.array_equal(out_bits[plain], bits_in[src_rows[plain]]), f"slab {s}: {name} copies not bit-exact"
        if merged.any():
            got = widen(out_bits[merged])
            want = exact[merged]
            tol = np.abs(want) * 2.0 ** -7 + absmean[merged] * 2.0 ** -20 + 1e-30
            bad = np.abs(got - want) > tol
            assert not bad.any(), f"slab {s}: {name} centroid off by {np.abs(got - want)[bad].max()}"


def run_csm(k_bits, v_bits, deg, chunk, ns, nr, nm):
    k = to_dev(k_bits, "bf16")
    v = to_dev(v_bits, "bf16")
    dg = None if deg is None else torch.from_numpy(np.ascontiguousarray(deg, dtype=np.int32)).to(k.device)
    ko, vo, do, sc, mt, ch = K.kvsel_csm(k, v, dg, chunk=chunk, n_sink=ns, n_recent=nr, n_merge=nm,
                                         with_decisions=True)
    torch.cuda.synchronize()
    return {"k": to_host(ko), "v": to_host(vo), "degree": do.cpu().numpy(), "score": sc.cpu().numpy(),
            "match": mt.cpu().numpy(), "chosen": ch.cpu().numpy()}


def test_csm_chosen_token_without_partner():
    """A key with a NaN element gives its A token NaN similarities, so it has no
    partner (score -inf, match -1). With n_merge equal to the candidate count
    that token ranks in; the merge drops it instead of writing outside the
    span's LDS. The finite slab of the same call matches the oracle in full,
    and the other slab keeps n_out rows with the dropped token's degree gone."""
    n, d, chunk, ns, nr = 200, 128, 16, 2, 6
    wl = BATCHED.with_(name="csm_nan", wid=690, n_layers=1, batch=1, n_kv_heads=2, n_q_heads=2, head_dim=d,
                       n_keys=n, window=1, kv_budget=1)
    inp = make_inputs(wl)
    kb = inp["k"].reshape(2, n, d).copy()
    vb = inp["v"].reshape(2, n, d)
    bad = ns + 3 * chunk + 4          # an A position (even offset in its chunk) of slab 1
    kb[1, bad, 5] = 0x7FC0             # bf16 NaN
    nm = oracle_candidates(n, chunk, ns, nr)
    say("case csm nan key", n, chunk, nm)
    gpu = run_csm(kb.reshape(1, 1, 2, n, d), vb.reshape(1, 1, 2, n, d), None, chunk, ns, nr, nm)
    per = {key: gpu[key].reshape((2,) + gpu[key].shape[3:]) for key in gpu}
    ai = (bad - ns) // 2               # A number of the NaN token
    assert per["match"][1][ai] == -1 and np.isneginf(per["score"][1][ai])
    assert ai in per["chosen"][1].tolist()
    assert per["degree"][1].shape == (n - nm,)
    assert int(per["degree"][1].sum()) == n - 1   # every token but the dropped one is counted once
    check_csm_slab(kb[0], vb[0], np.ones(n, dtype=np.int64), chunk, ns, nr, nm,
                   {key: per[key][0] for key in per}, 0)


# (L, B, Hkv, n, d, chunk, n_sink, n_recent, rate)
CSM_CASES = [
    (1, 1, 2, 1000, 128, 64, 4, 32, 0.25),
    (1, 2, 2, 777, 64, 16, 1, 7, 0.4),     # d = 64, ragged last chunk
    (2, 1, 1, 513, 128, 2, 0, 0, 0.5),     # chunk 2: fixed pairs, every candidate merged
    (1, 1, 3, 301, 128, 8, 3, 5, 0.1),
    (1, 1, 2, 97, 128, 64, 0, 32, 0.3),    # one partial chunk
    (1, 1, 1, 66, 128, 64, 1, 0, 0.45),    # last chunk of length 1 (no candidate)
    (1, 1, 2, 40, 128, 8, 20, 20, 0.0),    # empty middle
]


@pytest.mark.parametrize("case", CSM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_csm_round(case):
    L, B, Hkv, n, d, chunk, ns, nr, rate = case
    say("case csm", case)
    wl = BATCHED.with_(name="csm", wid=600 + CSM_CASES.index(case), n_layers=L, batch=B, n_kv_heads=Hkv,
                       n_q_heads=Hkv, head_dim=d, n_keys=n, window=1, kv_budget=1)
    inp = make_inputs(wl)
    nm = min(K.csm_merge_count(rate, n, ns, nr), oracle_candidates(n, chunk, ns, nr))
    kb = inp["k"].reshape(-1, n, d)
    vb = inp["v"].reshape(-1, n, d)
    gpu = run_csm(inp["k"], inp["v"], None, chunk, ns, nr, nm)
    S = kb.shape[0]
    for s in range(S):
        sl = {key: val.reshape((S,) + val.shape[len(inp["k"].shape) - 2:])[s] for key, val in gpu.items()}
        check_csm_slab(kb[s], vb[s], np.ones(n, dtype=np.int64), chunk, ns, nr, nm, sl, s)


def oracle_candidates(n, chunk, ns, nr):
    _, a_pos = oracle.csm_layout(n, chunk, ns, nr)
    chunks, _ = oracle.csm_layout(n, chunk, ns, nr)
    return sum((e - s + 1) // 2 for (s, e) in chunks if e - s >= 2)


def test_csm_candidates_helper():
    for args in [(1000, 64, 4, 32), (66, 64, 1, 0), (40, 8, 20, 20), (513, 2, 0, 0), (777, 16, 1, 7)]:
        assert K.load_library().kvsel_csm_candidates(*args) == oracle_candidates(*args)


def test_csm_identical_keys_ties():
    """Constant keys: every similarity ties exactly on the GPU too, so each A
    token takes the first B token of its chunk and the lowest A tokens merge."""
    n, d, chunk, nm = 256, 128, 16, 40
    wl = BATCHED.with_(name="csm_const", wid=620, n_layers=1, batch=1, n_kv_heads=2, n_q_heads=2, n_keys=n,
                       window=1, kv_budget=1, key_model="const")
    say("case csm ties")
    inp = make_inputs(wl)
    gpu = run_csm(inp["k"], inp["v"], None, chunk, 0, 0, nm)
    for s in range(2):
        m = gpu["match"].reshape(2, -1)[s]
        a = np.arange(0, n, 2)
        assert m.tolist() == ((a // chunk) * chunk + 1).tolist()
        assert gpu["chosen"].reshape(2, -1)[s].tolist() == list(range(nm))


def test_csm_two_rounds_progressive():
    """Two rounds (rate 0.3 then 0.2): the second starts from the first's
    degrees; every round is checked on its own decisions."""
    n, d, chunk, ns, nr = 1200, 128, 32, 4, 64
    wl = BATCHED.with_(name="csm2", wid=621, n_layers=1, batch=1, n_kv_heads=2, n_q_heads=2, n_keys=n, window=1,
                       kv_budget=1)
    say("case csm two rounds")
    inp = make_inputs(wl)
    kb, vb = inp["k"].reshape(2, n, d), inp["v"].reshape(2, n, d)
    deg = np.ones((2, n), dtype=np.int64)
    for rate in (0.3, 0.2):
        nm = K.csm_merge_count(rate, kb.shape[1], ns, nr)
        gpu = run_csm(kb, vb, deg, chunk, ns, nr, nm)
        for s in range(2):
            sl = {key: val[s] for key, val in gpu.items()}
            check_csm_slab(kb[s], vb[s], deg[s], chunk, ns, nr, nm, sl, s)
        kb, vb, deg = gpu["k"], gpu["v"], gpu["degree"].astype(np.int64)
    assert (deg.sum(axis=1) == n).all()


def check_decode(q_bits, k_bits, v_bits, deg, out, scale):
    B, Hq, d = q_bits.shape
    for b in range(B):
        ref = oracle.decode_attention(widen(q_bits[b]), widen(k_bits[b]), widen(v_bits[b]),
                                      None if deg is None else deg[b], scale)
        vmax = np.abs(widen(v_bits[b])).max()
        err = np.abs(out[b].astype(np.float64) - ref)
        tol = 1e-4 * vmax + 1e-4 * np.abs(ref)
        assert (err <= tol).all(), f"decode b={b}: max err {err.max()} (tol {tol.max()})"


# (B, Hq, Hkv, n, d, with degrees)
DEC_CASES = [
    (2, 8, 2, 1000, 128, False),
    (1, 28, 4, 4096, 128, True),   # G = 7
    (3, 4, 4, 63, 64, False),      # fewer keys than one block, d = 64
    (1, 32, 8, 5000, 128, True),
    (2, 2, 2, 1, 128, False),      # a single key
    (1, 8, 1, 70000, 64, True),    # many splits, G = 8
    (2, 6, 2, 3001, 128, True),    # G = 3 (8 rows per lane), ragged
    (1, 16, 4, 33, 128, True),     # G = 4, fewer keys than one 8-row block per wave
    (1, 4, 2, 4100, 128, False),   # G = 2
    (1, 10, 2, 777, 128, False),   # G = 5
    (2, 12, 2, 2049, 128, True),   # G = 6
    (1, 16, 2, 1500, 128, True),   # G = 8
]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_attention(case):
    B, Hq, Hkv, n, d, with_deg = case
    say("case decode", case)
    rng = np.random.default_rng(700 + DEC_CASES.index(case))
    def bf16_bits(x):
        return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = bf16_bits(rng.normal(size=(B, Hq, d)))
    k = bf16_bits(rng.normal(size=(B, Hkv, n, d)) * 1.5)
    v = bf16_bits(rng.normal(size=(B, Hkv, n, d)))
    deg = rng.integers(1, 20, size=(B, Hkv, n)).astype(np.int32) if with_deg else None
    out = K.kvsel_decode_attention(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                   None if deg is None else torch.from_numpy(deg).cuda())
    torch.cuda.synchronize()
    check_decode(q, k, v, deg, out.cpu().numpy(), 1.0 / math.sqrt(d))


def test_decode_duplicates_equal_degrees():
    """Attention over a cache with duplicated rows equals attention over the
    deduplicated cache with the multiplicities as degrees (the log term)."""
    rng = np.random.default_rng(731)
    d, n = 128, 300
    def bf16_bits(x):
        return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = bf16_bits(rng.normal(size=(1, 4, d)))
    k = bf16_bits(rng.normal(size=(1, 1, n, d)))
    v = bf16_bits(rng.normal(size=(1, 1, n, d)))
    mult = rng.integers(1, 4, size=n)
    kx = np.repeat(k, mult, axis=2)
    vx = np.repeat(v, mult, axis=2)
    dev = lambda a: to_dev(np.ascontiguousarray(a), "bf16")
    o1 = K.kvsel_decode_attention(dev(q), dev(kx), dev(vx)).cpu().numpy()
    o2 = K.kvsel_decode_attention(dev(q), dev(k), dev(v),
                                  torch.from_numpy(mult.astype(np.int32).reshape(1, 1, n)).cuda()).cpu().numpy()
    np.testing.assert_allclose(o1, o2, rtol=1e-4, atol=1e-5)


def test_full_size_csm_and_decode():
    """The batched 8 x 32K workload (AR(1) keys, 8 x 8 slabs): one CSM round at
    rate 0.25 (chunk 64, 4 sinks, 32 recent tokens) checked on two sampled
    slabs; then a decode step over the compacted cache with degrees, checked
    for every sequence against the oracle on the GPU's compacted cache."""
    wl = BATCHED
    t0 = time.time()
    say("case full csm: inputs")
    inp = make_inputs(wl, with_hidden=False, threads=16)
    n, d, chunk, ns, nr = wl.n_keys, wl.head_dim, 64, 4, 32
    nm = K.csm_merge_count(0.25, n, ns, nr)
    say(f"case full csm: HIP ({time.time() - t0:.1f}s)")
    gpu = run_csm(inp["k"], inp["v"], None, chunk, ns, nr, nm)
    S = wl.n_layers * wl.batch * wl.n_kv_heads
    kb = inp["k"].reshape(S, n, d)
    vb = inp["v"].reshape(S, n, d)
    for s in (0, S - 1):
        say(f"case full csm: oracle slab {s} ({time.time() - t0:.1f}s)")
        sl = {key: val.reshape((S,) + val.shape[3:])[s] for key, val in gpu.items()}
        check_csm_slab(kb[s], vb[s], np.ones(n, dtype=np.int64), chunk, ns, nr, nm, sl, s)
    say(f"case full csm: decode ({time.time() - t0:.1f}s)")
    B, Hq, Hkv = wl.batch, wl.n_q_heads, wl.n_kv_heads
    q = inp["q"][0][:, :, -1]  # the last window query of every head: [B, Hq, d]
    kc = gpu["k"].reshape(B, Hkv, n - nm, d)
    vc = gpu["v"].reshape(B, Hkv, n - nm, d)
    dc = gpu["degree"].reshape(B, Hkv, n - nm)
    out = K.kvsel_decode_attention(to_dev(np.ascontiguousarray(q), "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"),
                                   torch.from_numpy(dc.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    check_decode(np.ascontiguousarray(q), kc, vc, dc, out.cpu().numpy(), 1.0 / math.sqrt(d))
    say(f"case full csm: done ({time.time() - t0:.1f}s)")
