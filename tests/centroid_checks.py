"""Pins of the CentroidKV / decode-attention oracle (oracle/centroid_oracle.py)
to facts fixed outside it: a loop brute force written separately, closed
forms, invariants. Each check takes the oracle module (or a planted-mistake
copy of it)."""

import math

import numpy as np


def _brute_csm(k, v, deg, chunk, n_sink, n_recent, n_merge):
    """Lists and loops: partition, cosine best match (ties to the lower B),
    rank (similarity desc, A position asc), merge into weighted means."""
    n, d = len(k), len(k[0])
    lo, hi = n_sink, n - n_recent
    cands = []  # (similarity, a, b)
    for s in range(lo, hi, chunk):
        e = min(s + chunk, hi)
        for a in range(s, e, 2):
            best = None
            for b in range(s + 1, e, 2):
                na = math.sqrt(math.fsum(x * x for x in k[a]))
                nb = math.sqrt(math.fsum(x * x for x in k[b]))
                c = 0.0 if na == 0 or nb == 0 else math.fsum(x * y for x, y in zip(k[a], k[b])) / (na * nb)
                if best is None or c > best[0]:
                    best = (c, b)
            if best is not None:
                cands.append((best[0], a, best[1]))
    cands.sort(key=lambda t: (-t[0], t[1]))
    chosen = cands[:n_merge]
    members = {j: [j] for j in range(n)}
    for _, a, b in chosen:
        members[b].append(a)
        del members[a]
    out_k, out_v, out_d = [], [], []
    for j in sorted(members):
        mem = members[j]
        w = math.fsum(deg[i] for i in mem)
        out_k.append([math.fsum(deg[i] * k[i][t] for i in mem) / w for t in range(d)])
        out_v.append([math.fsum(deg[i] * v[i][t] for i in mem) / w for t in range(d)])
        out_d.append(int(w))
    return out_k, out_v, out_d, sorted((a, b) for _, a, b in chosen)


def check_csm_brute(orc):
    """csm_round == the loop brute force on small slabs: ragged last chunks,
    sinks and recent tokens, degrees above one, chunk 2 and 8."""
    rng = np.random.default_rng(201)
    for (n, d, chunk, ns, nr, nm) in [(23, 4, 4, 2, 3, 5), (30, 3, 8, 0, 0, 9), (17, 5, 2, 1, 1, 6),
                                      (12, 2, 6, 3, 2, 0), (40, 4, 8, 4, 4, 14)]:
        base = rng.normal(size=(n, d))
        k = np.cumsum(base, axis=0) * 0.3 + base  # locally similar keys
        v = rng.normal(size=(n, d))
        deg = rng.integers(1, 5, size=n)
        r = orc.csm_round(k, v, deg, chunk, ns, nr, nm)
        bk, bv, bd, pairs = _brute_csm(k.tolist(), v.tolist(), deg.tolist(), chunk, ns, nr, nm)
        np.testing.assert_allclose(r["k"], np.array(bk), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["v"], np.array(bv), rtol=1e-12, atol=1e-12)
        assert r["degree"].tolist() == bd
        got = sorted((int(r["a_pos"][i]), int(r["match"][i])) for i in r["chosen"])
        assert got == pairs


def check_csm_invariants(orc):
    """Degrees and degree-weighted sums of keys and values are conserved; the
    cache shrinks by exactly n_merge; sinks and recent tokens are untouched;
    n_merge = 0 is the identity; merge_count's closed form."""
    rng = np.random.default_rng(202)
    n, d, chunk, ns, nr, nm = 64, 6, 8, 3, 5, 20
    k = rng.normal(size=(n, d))
    v = rng.normal(size=(n, d))
    deg = rng.integers(1, 9, size=n)
    r = orc.csm_round(k, v, deg, chunk, ns, nr, nm)
    assert r["k"].shape == (n - nm, d) and r["degree"].sum() == deg.sum()
    np.testing.assert_allclose((r["k"] * r["degree"][:, None]).sum(0), (k * deg[:, None]).sum(0), rtol=1e-12)
    np.testing.assert_allclose((r["v"] * r["degree"][:, None]).sum(0), (v * deg[:, None]).sum(0), rtol=1e-12)
    np.testing.assert_array_equal(r["k"][:ns], k[:ns])
    np.testing.assert_array_equal(r["k"][-nr:], k[-nr:])
    np.testing.assert_array_equal(r["degree"][-nr:], deg[-nr:])
    r0 = orc.csm_round(k, v, deg, chunk, ns, nr, 0)
    np.testing.assert_array_equal(r0["k"], k)
    np.testing.assert_array_equal(r0["degree"], deg)
    assert orc.merge_count(0.25, 1000, 4, 32) == 241 and orc.merge_count(0.0, 10, 0, 0) == 0


def check_csm_ties_and_pairs(orc):
    """Identical keys: every similarity ties, so each A token takes the first B
    token of its chunk and the lowest A positions are merged. Chunk 2: each A
    token's only candidate is the next position. Orthogonal keys score 0, a
    zero key scores 0 (cosine convention)."""
    n, d = 20, 4
    k = np.tile(np.array([1.0, 2.0, -1.0, 0.5]), (n, 1))
    v = np.arange(n * d, dtype=np.float64).reshape(n, d)
    r = orc.csm_round(k, v, None, 4, 0, 0, 3)
    assert r["match"].tolist() == [1, 1, 5, 5, 9, 9, 13, 13, 17, 17]
    assert r["chosen"].tolist() == [0, 1, 2]  # A positions 0, 2, 4
    assert r["degree"].tolist()[:3] == [3, 1, 2]  # survivors 1 = {0, 1, 2}, 3, 5 = {4, 5}
    np.testing.assert_allclose(r["v"][0], (v[0] + v[1] + v[2]) / 3)
    a_pos, score, match = orc.csm_match(np.random.default_rng(3).normal(size=(9, 3)), 2, 0, 0)
    assert match.tolist() == [1, 3, 5, 7, -1] and np.isneginf(score[-1])
    e = np.eye(4)
    _, s2, _ = orc.csm_match(np.stack([e[0], e[1], np.zeros(4), e[2]]), 4, 0, 0)
    assert s2.tolist() == [0.0, 0.0]


def check_decode_attention(orc):
    """Degree-one attention == softmax by loops; q = 0 gives the degree-weighted
    mean of the values; attention over a cache of duplicated tokens equals
    attention over its compacted form with degrees (the log term's purpose)."""
    rng = np.random.default_rng(203)
    Hq, Hkv, n, d = 4, 2, 7, 5
    q = rng.normal(size=(Hq, d))
    k = rng.normal(size=(Hkv, n, d))
    v = rng.normal(size=(Hkv, n, d))
    out = orc.decode_attention(q, k, v, None, 0.4)
    for h in range(Hq):
        g = h // 2
        lg = [0.4 * math.fsum(q[h][t] * k[g][j][t] for t in range(d)) for j in range(n)]
        mx = max(lg)
        w = [math.exp(x - mx) for x in lg]
        ref = [math.fsum(w[j] * v[g][j][t] for j in range(n)) / math.fsum(w) for t in range(d)]
        np.testing.assert_allclose(out[h], ref, rtol=1e-12, atol=1e-13)
    deg = rng.integers(1, 6, size=(Hkv, n))
    o0 = orc.decode_attention(np.zeros((Hq, d)), k, v, deg, 0.4)
    for h in range(Hq):
        g = h // 2
        np.testing.assert_allclose(o0[h], (deg[g][:, None] * v[g]).sum(0) / deg[g].sum(), rtol=1e-12)
    for g in range(Hkv):  # head by head: the expanded caches differ in length
        kx = np.repeat(k[g], deg[g], axis=0)[None]
        vx = np.repeat(v[g], deg[g], axis=0)[None]
        qh = q[g * 2:(g + 1) * 2]
        np.testing.assert_allclose(orc.decode_attention(qh, kx, vx, None, 0.4),
                                   orc.decode_attention(qh, k[g:g + 1], v[g:g + 1], deg[g:g + 1], 0.4),
                                   rtol=1e-12, atol=1e-13)


CENTROID_CHECKS = [
    check_csm_brute,
    check_csm_invariants,
    check_csm_ties_and_pairs,
    check_decode_attention,
]
