"""Pure-Python brute force for tiny inputs: an implementation of the saliency
score that shares nothing with the oracle (explicit loops, math.exp,
math.fsum, per-row softmax written out), used to pin the oracle.

The score is the observation-window attention received by each key: window
query i of head h sits at position N - w + i, attends causally, and each KV
head's score is the mean over its G query heads of the window-summed softmax
(FastKV section 2A saliency; StructKV section 1 attention scores).
"""

from __future__ import annotations

import math


def brute_saliency(q, k, scale):
    """q: [Hq][w][d], k: [Hkv][N][d] (nested sequences of floats).

    Returns (lse[Hq][w], raw[Hkv][N]) as nested lists of floats.
    """
    Hq, w, d = len(q), len(q[0]), len(q[0][0])
    Hkv, N = len(k), len(k[0])
    G = Hq // Hkv
    lse = [[0.0] * w for _ in range(Hq)]
    raw = [[0.0] * N for _ in range(Hkv)]
    for h in range(Hq):
        g = h // G
        for i in range(w):
            pos = N - w + i
            logit = []
            for j in range(pos + 1):
                logit.append(scale * math.fsum(q[h][i][t] * k[g][j][t] for t in range(d)))
            top = max(logit)
            weights = [math.exp(x - top) for x in logit]
            total = math.fsum(weights)
            lse[h][i] = top + math.log(total)
            for j in range(pos + 1):
                raw[g][j] += weights[j] / total / G
    return lse, raw


def brute_saliency_given_lse(q, k, lse, scale):
    """As brute_saliency, with each window row's natural-log LSE given
    (lse[Hq][w]) instead of computed: raw[g][j] = sum over the group's rows of
    exp(logit - lse) / G."""
    Hq, w, d = len(q), len(q[0]), len(q[0][0])
    Hkv, N = len(k), len(k[0])
    G = Hq // Hkv
    raw = [[0.0] * N for _ in range(Hkv)]
    for h in range(Hq):
        g = h // G
        for i in range(w):
            for j in range(N - w + i + 1):
                logit = scale * math.fsum(q[h][i][t] * k[g][j][t] for t in range(d))
                raw[g][j] += math.exp(logit - lse[h][i]) / G
    return raw


def brute_pool(x, kernel):
    """Average pool, zero padded, divisor always ``kernel``."""
    r = (kernel - 1) // 2
    n = len(x)
    out = []
    for j in range(n):
        acc = []
        for t in range(j - r, j + r + 1):
            acc.append(x[t] if 0 <= t < n else 0.0)
        out.append(math.fsum(acc) / kernel)
    return out


def brute_select(score, n_keys, window, budget):
    """Largest (budget - window) scores, ties to the lower position, plus the
    window; ascending."""
    n_prefix = n_keys - window
    ranked = sorted(range(n_prefix), key=lambda j: (-score[j], j))
    kept = sorted(ranked[: budget - window]) + list(range(n_prefix, n_keys))
    return kept


def brute_max_pool(x, kernel):
    """Max over the positions j - r .. j + r inside the row."""
    r = (kernel - 1) // 2
    n = len(x)
    return [max(x[t] for t in range(max(0, j - r), min(n, j + r + 1))) for j in range(n)]


def brute_select_sinks(score, n_keys, window, budget, n_sink):
    """Positions 0 .. n_sink-1, then the largest (budget - window - n_sink)
    scores of the other prefix positions (ties to the lower position), plus
    the window; ascending."""
    n_prefix = n_keys - window
    rest = sorted(range(n_sink, n_prefix), key=lambda j: (-score[j], j))
    return sorted(list(range(n_sink)) + rest[: budget - window - n_sink]) + list(range(n_prefix, n_keys))


def brute_row_stats(q, k, scale, small_p):
    """Per window row: entropy -sum p ln p, sum p^2 and the count of visible
    keys with p < small_p, by explicit loops (q [Hq][w][d], k [Hkv][N][d])."""
    Hq, w, d = len(q), len(q[0]), len(q[0][0])
    Hkv, N = len(k), len(k[0])
    G = Hq // Hkv
    ent = [[0.0] * w for _ in range(Hq)]
    sp2 = [[0.0] * w for _ in range(Hq)]
    nb = [[0] * w for _ in range(Hq)]
    for h in range(Hq):
        for i in range(w):
            logit = [scale * math.fsum(q[h][i][t] * k[h // G][j][t] for t in range(d)) for j in range(N - w + i + 1)]
            top = max(logit)
            total = math.fsum(math.exp(x - top) for x in logit)
            probs = [math.exp(x - top) / total for x in logit]
            ent[h][i] = -math.fsum(pj * math.log(pj) for pj in probs if pj > 0.0)
            sp2[h][i] = math.fsum(pj * pj for pj in probs)
            nb[h][i] = sum(1 for pj in probs if pj < small_p)
    return ent, sp2, nb
