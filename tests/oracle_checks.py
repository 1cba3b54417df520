"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``check_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with something fixed independently of it: a brute force
written separately, a closed form, a library routine, or an invariant of the
definition. The pin tests run them on the real oracle (all must pass); the
mutation tests run them on copies of the oracle with a planted mistake (at
least one must fail).
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp

from brute_force import (brute_max_pool, brute_pool, brute_row_stats, brute_saliency, brute_saliency_given_lse,
                         brute_select, brute_select_sinks)

# tiny shapes: (Hq, Hkv, w, d, N, pool, budget)
TINY_CASES = [
    (1, 1, 1, 4, 9, 1, 3),
    (2, 1, 2, 4, 13, 3, 5),
    (4, 2, 4, 8, 24, 7, 10),
    (6, 2, 3, 5, 21, 3, 8),      # G = 3, odd d
    (8, 2, 8, 8, 40, 7, 16),
    (4, 4, 2, 6, 17, 1, 2),      # G = 1, budget = w
    (3, 1, 5, 4, 16, 5, 16),     # budget = N
    (2, 2, 7, 4, 7, 1, 7),       # w = N: empty prefix
]


def _rand_case(rng, Hq, Hkv, w, d, N):
    q = rng.standard_normal((Hq, w, d))
    k = rng.standard_normal((Hkv, N, d))
    return q, k


def check_brute_force(orc):
    """Oracle == pure-Python brute force on tiny random inputs (scores, LSE,
    pooled scores, kept indices)."""
    rng = np.random.default_rng(1234)
    for (Hq, Hkv, w, d, N, pool, budget) in TINY_CASES:
        q, k = _rand_case(rng, Hq, Hkv, w, d, N)
        lse, raw = orc.saliency_one(q, k)
        blse, braw = brute_saliency(q.tolist(), k.tolist(), 1.0 / math.sqrt(d))
        np.testing.assert_allclose(lse, np.array(blse), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(raw, np.array(braw), rtol=1e-11, atol=1e-15)
        s = orc.pooled_scores(raw, w, pool)
        assert s.shape == (Hkv, N - w)
        for g in range(Hkv):
            bs = brute_pool(braw[g][: N - w], pool) if N > w else []
            np.testing.assert_allclose(s[g], np.array(bs), rtol=1e-11, atol=1e-15)
            kept = orc.select_row(s[g], N, w, budget)
            assert list(kept) == brute_select(list(s[g]), N, w, budget)


def check_pipeline_brute(orc):
    """Whole path over two layers and a TSP token set against the brute force:
    per-layer brute scores, pooled, summed over layers, head-mean, selected,
    gathered."""
    rng = np.random.default_rng(99)
    L, B, Hq, Hkv, w, d, N, pool, kvb, tspb = 2, 2, 4, 2, 3, 4, 20, 3, 8, 11
    q = rng.standard_normal((L, B, Hq, w, d)).astype(np.float32)
    k = rng.standard_normal((L, B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((L, B, Hkv, N, d)).astype(np.float32)
    hid = rng.standard_normal((B, N, 5)).astype(np.float32)
    out = orc.pipeline(q, k, v, dtype="f32", window=w, pool_kernel=pool, kv_budget=kvb,
                       tsp_budget=tspb, hidden=hid)
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        acc = [[0.0] * (N - w) for _ in range(Hkv)]
        for l in range(L):
            _, braw = brute_saliency(q[l, b].astype(np.float64).tolist(),
                                     k[l, b].astype(np.float64).tolist(), scale)
            for g in range(Hkv):
                ps = brute_pool(braw[g][: N - w], pool)
                acc[g] = [a + x for a, x in zip(acc[g], ps)]
        for g in range(Hkv):
            np.testing.assert_allclose(out["scores"][b, g], np.array(acc[g]), rtol=1e-11)
            kept = brute_select(acc[g], N, w, kvb)
            assert list(out["idx"][b, g]) == kept
            for l in range(L):
                for t, j in enumerate(kept):
                    assert out["k_kept"][l, b, g, t].tobytes() == k[l, b, g, j].tobytes()
                    assert out["v_kept"][l, b, g, t].tobytes() == v[l, b, g, j].tobytes()
        tsc = [sum(acc[g][j] for g in range(Hkv)) / Hkv for j in range(N - w)]
        np.testing.assert_allclose(out["tsp_scores"][b, 0], np.array(tsc), rtol=1e-11)
        tkept = brute_select(tsc, N, w, tspb)
        assert list(out["tsp_idx"][b, 0]) == tkept
        for t, j in enumerate(tkept):
            assert out["hidden_kept"][b, t].tobytes() == hid[b, j].tobytes()


def check_zero_query_closed_form(orc):
    """q = 0: every visible logit is 0, so window query i spreads 1/(p_i + 1)
    over its p_i + 1 visible keys. Prefix key j gets sum_i 1/(N - w + i + 1)
    = H_N - H_{N-w}; window key N - w + m gets sum_{i >= m} 1/(N - w + i + 1)."""
    for (Hq, Hkv, w, d, N) in [(4, 2, 8, 16, 64), (3, 1, 1, 4, 10), (2, 2, 5, 8, 5)]:
        q = np.zeros((Hq, w, d))
        k = np.random.default_rng(5).standard_normal((Hkv, N, d))
        lse, raw = orc.saliency_one(q, k)
        Np = N - w
        harm = sum(1.0 / (Np + i + 1) for i in range(w))
        for g in range(Hkv):
            np.testing.assert_allclose(raw[g, :Np], harm, rtol=1e-13)
            for m in range(w):
                exp_m = sum(1.0 / (Np + i + 1) for i in range(m, w))
                np.testing.assert_allclose(raw[g, Np + m], exp_m, rtol=1e-13)
        for i in range(w):
            np.testing.assert_allclose(lse[:, i], math.log(Np + i + 1), rtol=1e-14)


def check_mass(orc):
    """Each window row's softmax sums to one, so each KV head's raw score sums
    to w over all N keys; every raw score is in [0, w]."""
    rng = np.random.default_rng(7)
    for (Hq, Hkv, w, d, N) in [(8, 2, 32, 16, 300), (6, 3, 4, 8, 50), (4, 4, 1, 4, 3)]:
        q, k = _rand_case(rng, Hq, Hkv, w, d, N)
        lse, raw = orc.saliency_one(q, k)
        np.testing.assert_allclose(raw.sum(axis=1), w, rtol=1e-12)
        assert (raw >= 0).all() and (raw <= w + 1e-12).all()


def check_lse_library(orc):
    """LSE equals scipy.special.logsumexp over the visible logits, computed
    here with einsum and an explicit slice for the causal limit."""
    rng = np.random.default_rng(11)
    Hq, Hkv, w, d, N = 6, 2, 5, 16, 77
    q, k = _rand_case(rng, Hq, Hkv, w, d, N)
    lse, _ = orc.saliency_one(q, k)
    G = Hq // Hkv
    for h in range(Hq):
        for i in range(w):
            vis = k[h // G, : N - w + i + 1]
            l = np.einsum("d,jd->j", q[h, i], vis) / math.sqrt(d)
            assert abs(lse[h, i] - logsumexp(l)) < 1e-12 * max(1.0, abs(lse[h, i]))


def check_stability(orc):
    """Keys scaled by 500 push logits past +-1000, beyond where exp overflows
    even in float64: the oracle must stay finite (a max-shifted softmax) and
    still match logsumexp and the mass invariant."""
    rng = np.random.default_rng(13)
    Hq, Hkv, w, d, N = 4, 2, 4, 16, 60
    q, k = _rand_case(rng, Hq, Hkv, w, d, N)
    k = k * 500.0
    lse, raw = orc.saliency_one(q, k)
    assert np.isfinite(lse).all() and np.isfinite(raw).all()
    assert np.abs(lse).max() > 750
    np.testing.assert_allclose(raw.sum(axis=1), w, rtol=1e-12)
    G = Hq // Hkv
    l = np.einsum("d,jd->j", q[1, 0], k[1 // G, : N - w + 1]) / math.sqrt(d)
    assert abs(lse[1, 0] - logsumexp(l)) < 1e-12 * abs(lse[1, 0])


def check_pool(orc):
    """Average pool: a constant c stays c inside, is c (r + 1 + t) / k at
    distance t < r from an edge, kernel 1 is the identity, and the result
    equals numpy.convolve with a box filter in 'same' mode."""
    for kern in (1, 3, 5, 7):
        r = (kern - 1) // 2
        c = 0.37
        x = np.full(40, c)
        s = orc.avg_pool(x, kern)
        np.testing.assert_allclose(s[r: 40 - r], c, rtol=1e-15)
        for t in range(r):
            np.testing.assert_allclose(s[t], c * (r + 1 + t) / kern, rtol=1e-15)
            np.testing.assert_allclose(s[39 - t], c * (r + 1 + t) / kern, rtol=1e-15)
        y = np.random.default_rng(kern).random(33)
        np.testing.assert_allclose(orc.avg_pool(y, kern),
                                   np.convolve(y, np.ones(kern) / kern, mode="same"), rtol=1e-14)
    np.testing.assert_array_equal(orc.avg_pool(np.arange(9.0), 1), np.arange(9.0))


def check_accumulate(orc):
    """StructKV accumulation is a plain sum over layers and the token-set
    score is a plain mean over KV heads; with one head the mean is that head."""
    rng = np.random.default_rng(17)
    per = rng.random((5, 2, 3, 11))
    acc = orc.accumulate_layers(per)
    ref = per[0] + per[1] + per[2] + per[3] + per[4]
    np.testing.assert_allclose(acc, ref, rtol=1e-15)
    hm = orc.head_mean(per[0])
    assert hm.shape == (2, 1, 11)
    np.testing.assert_allclose(hm[:, 0], (per[0][:, 0] + per[0][:, 1] + per[0][:, 2]) / 3, rtol=1e-15)
    one = per[0][:, :1]
    np.testing.assert_array_equal(orc.head_mean(one), one)


def check_select(orc):
    """Kept set against the brute force on scores with many exact ties, and the
    invariants: exactly ``budget`` indices, strictly ascending, the window is
    the last w entries, every kept prefix score >= every dropped one."""
    rng = np.random.default_rng(19)
    for trial in range(40):
        N = int(rng.integers(1, 60))
        w = int(rng.integers(1, N + 1))
        budget = int(rng.integers(w, N + 1))
        s = rng.integers(0, 5, size=N - w).astype(np.float64)  # heavy ties
        kept = orc.select_row(s, N, w, budget)
        assert list(kept) == brute_select(list(s), N, w, budget)
        assert len(kept) == budget
        assert np.all(np.diff(kept) > 0)
        assert list(kept[budget - w:]) == list(range(N - w, N))
        pre = kept[: budget - w]
        dropped = np.setdiff1d(np.arange(N - w), pre)
        if pre.size and dropped.size:
            assert s[pre].min() >= s[dropped].max()


def check_tie_pin(orc):
    """q = 0 makes every prefix raw score bit-identical, so the tie-break alone
    decides: kernel 1 keeps [0, kk) and the window; kernel 7 pushes the three
    positions at each edge down (zero padding), keeping [3, kk + 3)."""
    Hq, Hkv, w, d, N, budget = 4, 2, 8, 16, 200, 40
    kk = budget - w
    q = np.zeros((Hq, w, d))
    k = np.random.default_rng(3).standard_normal((Hkv, N, d))
    _, raw = orc.saliency_one(q, k)
    s1 = orc.pooled_scores(raw, w, 1)
    s7 = orc.pooled_scores(raw, w, 7)
    for g in range(Hkv):
        assert list(orc.select_row(s1[g], N, w, budget)) == list(range(kk)) + list(range(N - w, N))
        assert list(orc.select_row(s7[g], N, w, budget)) == list(range(3, kk + 3)) + list(range(N - w, N))


def check_causal(orc):
    """A key after window query i's position cannot change that row's LSE;
    changing the last key changes only the last row."""
    rng = np.random.default_rng(23)
    Hq, Hkv, w, d, N = 2, 1, 4, 8, 30
    q, k = _rand_case(rng, Hq, Hkv, w, d, N)
    lse0, _ = orc.saliency_one(q, k)
    k2 = k.copy()
    k2[:, N - 1] += 5.0
    lse1, _ = orc.saliency_one(q, k2)
    np.testing.assert_array_equal(lse0[:, : w - 1], lse1[:, : w - 1])
    assert np.all(lse0[:, w - 1] != lse1[:, w - 1])


def check_gqa_map(orc):
    """Query head h reads KV head floor(h / G): changing the keys of KV head 1
    changes the LSE of query heads G .. 2G - 1 only."""
    rng = np.random.default_rng(29)
    Hq, Hkv, w, d, N = 6, 2, 3, 8, 25
    q, k = _rand_case(rng, Hq, Hkv, w, d, N)
    lse0, raw0 = orc.saliency_one(q, k)
    k2 = k.copy()
    k2[1] *= 1.5
    lse1, raw1 = orc.saliency_one(q, k2)
    np.testing.assert_array_equal(lse0[:3], lse1[:3])
    assert np.all(lse0[3:] != lse1[3:])
    np.testing.assert_array_equal(raw0[0], raw1[0])


def check_gather(orc):
    """Gathered rows are bit-identical to the source rows at the kept index,
    for any bit pattern (NaN payloads included)."""
    rng = np.random.default_rng(31)
    src = rng.integers(0, 1 << 16, size=(3, 50, 7), dtype=np.uint16)
    idx = np.stack([np.sort(rng.choice(50, 12, replace=False)) for _ in range(3)])
    out = orc.gather_rows(src, idx)
    for p in range(3):
        for t in range(12):
            assert out[p, t].tobytes() == src[p, idx[p, t]].tobytes()
    shared = orc.gather_rows(src, idx[:1])
    for p in range(3):
        for t in range(12):
            assert shared[p, t].tobytes() == src[p, idx[0, t]].tobytes()


def check_widening(orc):
    """bf16 bit patterns widen exactly: 0x3F80 is 1.0, 0xC000 is -2.0, 0x3EAB
    is 0.333984375, 0x0001 is the smallest subnormal 2^-133."""
    bits = np.array([0x3F80, 0xC000, 0x3EAB, 0x0001], dtype=np.uint16)
    out = orc.to_f64(bits, "bf16")
    assert list(out) == [1.0, -2.0, 0.333984375, 2.0 ** -133]


def check_given_lse_brute(orc):
    """Scores from a handed-in LSE == the separately written brute force, for
    LSE values away from the true ones (random offsets per row)."""
    rng = np.random.default_rng(77)
    for (Hq, Hkv, w, d, N, pool, budget) in TINY_CASES:
        q, k = _rand_case(rng, Hq, Hkv, w, d, N)
        lse = rng.normal(2.0, 1.5, size=(Hq, w))
        raw = orc.saliency_given_lse(q, k, lse)
        braw = brute_saliency_given_lse(q.tolist(), k.tolist(), lse.tolist(), 1.0 / math.sqrt(d))
        np.testing.assert_allclose(raw, np.array(braw), rtol=1e-11, atol=1e-15)


def check_given_lse_mass_and_shift(orc):
    """With the true LSE (scipy's logsumexp over the visible logits, computed
    here) every row's probabilities sum to one, so each KV head's raw scores
    sum to w; adding delta to every row's LSE scales every score by
    exp(-delta)."""
    rng = np.random.default_rng(78)
    for (Hq, Hkv, w, d, N, pool, budget) in TINY_CASES:
        q, k = _rand_case(rng, Hq, Hkv, w, d, N)
        G = Hq // Hkv
        scale = 1.0 / math.sqrt(d)
        lse = np.empty((Hq, w))
        for h in range(Hq):
            for i in range(w):
                vis = k[h // G, : N - w + i + 1] @ q[h, i] * scale
                lse[h, i] = logsumexp(vis)
        raw = orc.saliency_given_lse(q, k, lse)
        np.testing.assert_allclose(raw.sum(axis=1), np.full(Hkv, float(w)), rtol=1e-12)
        delta = 0.731
        np.testing.assert_allclose(orc.saliency_given_lse(q, k, lse + delta), raw * math.exp(-delta),
                                   rtol=1e-12, atol=1e-300)


def _bf16_bits(x):
    """Round float64 values to bf16 (nearest-even) and return the bit patterns."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _bits_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_all_drivers_per_slice(orc):
    """The per-(layer, sequence) drivers saliency_all_given_lse and
    row_stats_all against the brute force of each slice: L = 2, B = 2 with
    inputs that differ in every (l, b) (and LSE offsets that differ per row),
    bf16 and fp32 storage, one worker thread and two. A swapped l/b index or
    a wrong slice puts another slice's numbers in place and fails here."""
    rng = np.random.default_rng(4321)
    L, B, Hq, Hkv, w, d, N, tau = 2, 2, 4, 2, 3, 4, 11, 0.08
    scale = 1.0 / math.sqrt(d)
    for dtype in ("bf16", "f32"):
        qf = rng.standard_normal((L, B, Hq, w, d)) * (1.0 + np.arange(L * B).reshape(L, B, 1, 1, 1))
        kf = rng.standard_normal((L, B, Hkv, N, d)) + 0.3 * np.arange(L * B).reshape(L, B, 1, 1, 1)
        if dtype == "bf16":
            q, k = _bf16_bits(qf), _bf16_bits(kf)
            qv, kv = _bits_to_f64(q), _bits_to_f64(k)
        else:
            q, k = qf.astype(np.float32), kf.astype(np.float32)
            qv, kv = q.astype(np.float64), k.astype(np.float64)
        lse = rng.normal(1.5, 1.0, size=(L, B, Hq, w)) + np.arange(L * B).reshape(L, B, 1, 1)
        for threads in (1, 2):
            raw = orc.saliency_all_given_lse(q, k, lse, dtype, threads=threads)
            ent, sp2, nb = orc.row_stats_all(q, k, dtype, tau, threads=threads)
            assert raw.shape == (L, B, Hkv, N) and ent.shape == sp2.shape == nb.shape == (L, B, Hq, w)
            for l in range(L):
                for b in range(B):
                    braw = brute_saliency_given_lse(qv[l, b].tolist(), kv[l, b].tolist(), lse[l, b].tolist(),
                                                    scale)
                    np.testing.assert_allclose(raw[l, b], np.array(braw), rtol=1e-11, atol=1e-15)
                    bent, bsp2, bnb = brute_row_stats(qv[l, b].tolist(), kv[l, b].tolist(), scale, tau)
                    np.testing.assert_allclose(ent[l, b], np.array(bent), rtol=1e-12, atol=1e-14)
                    np.testing.assert_allclose(sp2[l, b], np.array(bsp2), rtol=1e-12, atol=1e-14)
                    assert nb[l, b].tolist() == bnb


def check_max_pool(orc):
    """Max-pool variant: == the brute force on random rows; a lone spike of
    height h in a zero row becomes h on the 2r+1 positions around it (clipped
    at the ends) and 0 elsewhere; the pool never lowers a value."""
    rng = np.random.default_rng(79)
    for n in (1, 2, 5, 17, 40):
        for kernel in (1, 3, 5, 7, 9):
            x = rng.random(n)
            np.testing.assert_array_equal(orc.max_pool(x, kernel), np.array(brute_max_pool(list(x), kernel)))
            assert np.all(orc.max_pool(x, kernel) >= x)
    r, n = 3, 30
    for p in (0, 1, 14, 28, 29):
        x = np.zeros(n)
        x[p] = 2.5
        exp = np.zeros(n)
        exp[max(0, p - r):min(n, p + r + 1)] = 2.5
        np.testing.assert_array_equal(orc.max_pool(x, 2 * r + 1), exp)
    raw = rng.random((2, 3, 50))
    np.testing.assert_array_equal(orc.pooled_scores(raw, 6, 5, "max"), orc.max_pool(raw[..., :44], 5))


def check_sinks(orc):
    """Sink protection: == the brute force; every sink is kept even with the
    lowest scores; n_sink = 0 is the plain select."""
    rng = np.random.default_rng(80)
    for (N, w, budget, n_sink) in [(20, 3, 9, 2), (40, 5, 20, 15), (12, 2, 5, 3), (9, 1, 9, 8), (30, 4, 10, 0)]:
        score = rng.random(N - w)
        score[:n_sink] = 0.0  # sinks with the lowest scores
        kept = orc.select_row(score, N, w, budget, n_sink)
        assert list(kept) == brute_select_sinks(list(score), N, w, budget, n_sink)
        assert set(range(n_sink)) <= set(kept.tolist())
        if n_sink == 0:
            assert list(kept) == brute_select(list(score), N, w, budget)


def check_row_stats_brute(orc):
    """Row statistics == explicit loops on tiny shapes (G = 2, causal rows of
    different lengths), with the threshold between the rows' probabilities."""
    rng = np.random.default_rng(91)
    for (Hq, Hkv, w, N, d, tau) in [(2, 1, 3, 7, 4, 0.1), (4, 2, 4, 9, 3, 0.05), (3, 3, 1, 5, 2, 0.3)]:
        q = rng.normal(size=(Hq, w, d)) * 1.5
        k = rng.normal(size=(Hkv, N, d))
        ent, sp2, nb = orc.row_stats(q, k, tau)
        bent, bsp2, bnb = brute_row_stats(q.tolist(), k.tolist(), 1.0 / math.sqrt(d), tau)
        np.testing.assert_allclose(ent, np.array(bent), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sp2, np.array(bsp2), rtol=1e-12, atol=1e-14)
        assert nb.tolist() == bnb


def check_row_stats_closed_forms(orc):
    """q = 0: every row is uniform over its n_i visible keys, so entropy =
    ln n_i, sum p^2 = 1 / n_i, and n_below is n_i or 0 as the threshold lies
    above or below 1 / n_i. A dominant key: entropy -> 0 and sum p^2 -> 1.
    scipy.stats.entropy on one row. Bounds: -ln sum p^2 <= entropy <= ln n_i."""
    from scipy.stats import entropy as sp_entropy

    N, w, d = 40, 5, 8
    k = np.random.default_rng(92).normal(size=(2, N, d))
    n = N - w + 1 + np.arange(w)
    q = np.zeros((4, w, d))
    for tau, full in ((1.0 / (N - w + 1) + 1e-3, True), (1.0 / N - 1e-3, False)):
        ent, sp2, nb = orc.row_stats(q, k, tau)
        np.testing.assert_allclose(ent, np.broadcast_to(np.log(n), ent.shape), rtol=1e-13)
        np.testing.assert_allclose(sp2, np.broadcast_to(1.0 / n, sp2.shape), rtol=1e-12)
        assert (nb == (n if full else 0)).all()
    kd = np.zeros((1, N, d))
    kd[0, 3, 0] = 400.0
    qd = np.zeros((1, w, d))
    qd[0, :, 0] = 1.0
    ent, sp2, nb = orc.row_stats(qd, kd, 0.5)
    assert (ent < 1e-30 + 1e-10).all() and np.allclose(sp2, 1.0) and (nb == n - 1).all()
    rng = np.random.default_rng(93)
    q = rng.normal(size=(4, w, d)) * 2.0
    ent, sp2, nb = orc.row_stats(q, k, 1e-3)
    logits = orc.window_logits(q[1], k[0], 1.0 / math.sqrt(d))
    pr = np.exp(logits[2] - logits[2][np.isfinite(logits[2])].max())
    pr = pr[np.isfinite(logits[2])]
    assert abs(ent[1, 2] - sp_entropy(pr / pr.sum())) < 1e-12
    assert (ent <= np.log(n) + 1e-12).all() and (-np.log(sp2) <= ent + 1e-12).all()


def check_layer_summary_and_pivot(orc):
    """layer_summary of uniform rows: entropy ln n, sparsity 1 or 0, variance
    0. pivot_layer on hand-made sequences: the first layer where both the
    relative entropy fall and the sparsity rise reach their thresholds; a fall
    alone or a rise alone is no pivot; none -> the last layer."""
    L, B, Hq, w, N = 3, 1, 2, 4, 20
    n = N - w + 1 + np.arange(w)
    ent = np.broadcast_to(np.log(n), (L, B, Hq, w)).copy()
    sp2 = np.broadcast_to(1.0 / n, (L, B, Hq, w)).copy()
    nb = np.broadcast_to(n, (L, B, Hq, w)).copy()
    nb[1] = 0
    me, ms, mv = orc.layer_summary(ent, sp2, nb, N)
    np.testing.assert_allclose(me, np.log(n).mean())
    np.testing.assert_allclose(ms, [1.0, 0.0, 1.0])
    np.testing.assert_allclose(mv, 0.0, atol=1e-15)
    E = [10.0, 9.9, 9.8, 6.0, 5.9, 2.0]
    S = [0.10, 0.10, 0.12, 0.50, 0.52, 0.90]
    assert orc.pivot_layer(E, S, 0.1, 0.05) == 3
    assert orc.pivot_layer(E, S, 0.5, 0.05) == 5
    assert orc.pivot_layer(E, [0.1] * 6, 0.1, 0.05) == 5     # entropy falls, sparsity flat
    assert orc.pivot_layer([5.0] * 6, S, 0.1, 0.05) == 5     # sparsity rises, entropy flat
    assert orc.pivot_layer([10.0, 9.0, 8.9], [0.1, 0.3, 0.31], 0.05, 0.1) == 1
    assert orc.pivot_layer([10.0, 10.0, 5.0, 5.0], [0.0, 0.0, 0.5, 0.5], 0.1, 0.1) == 2
    assert orc.pivot_layer([10.0, 12.0, 5.0], [0.5, 0.0, 0.5], 0.1, 0.1) == 2  # rises are against l - 1
    assert orc.pivot_layer([7.0], [0.3], 0.1, 0.05) == 0


ALL_CHECKS = [
    check_all_drivers_per_slice,
    check_row_stats_brute,
    check_row_stats_closed_forms,
    check_layer_summary_and_pivot,
    check_max_pool,
    check_sinks,
    check_given_lse_brute,
    check_given_lse_mass_and_shift,
    check_brute_force,
    check_pipeline_brute,
    check_zero_query_closed_form,
    check_mass,
    check_lse_library,
    check_stability,
    check_pool,
    check_accumulate,
    check_select,
    check_tie_pin,
    check_causal,
    check_gqa_map,
    check_gather,
    check_widening,
]
