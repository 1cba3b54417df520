"""fp64 CPU oracle for CentroidKV's chunked soft matching (CSM) and for decode
attention over a compacted cache.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does, and it shares no code with the HIP kernels.

Source: the page "Technische Samenvatting: CentroidKV", section
"Methodologie", parts 2 (inference pipeline: sinks and recent tokens are
preserved before partitioning), 3 (chunked soft matching: chunks, alternating
A/B partition, best match across the sets, only the top fraction of matches
merged) and 4 (aggregation: degree-weighted centroids of keys and values, the
degree entering attention as a log term). The page gives no formulas; the
readings taken (all plain, all stated again in the functions) are:

* the middle of a slab is [n_sink, n - n_recent); chunk c covers middle
  positions [n_sink + c*C, n_sink + (c+1)*C) clipped to the middle;
* inside a chunk, offset 0, 2, 4, ... form set A and offset 1, 3, ... set B;
* similarity is the cosine of the two keys (0 when either key is zero);
  every A token's candidate is its most similar B token of the same chunk,
  ties to the lower position; an A token in a chunk without B tokens has no
  candidate;
* the n_merge candidates of highest similarity (ties to the lower A
  position) are merged, each into its B token; several A tokens may merge
  into one B token;
* a merged cluster's key and value are the degree-weighted means of its
  members, and its degree is the sum of theirs; tokens not merged are kept
  as they are; the compacted cache lists the survivors in position order;
* attention over a compacted cache adds ln(degree) to each key's logit.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np


def csm_layout(n: int, chunk: int, n_sink: int, n_recent: int):
    """Chunks of the middle region: a list of (start, end) positions, and the
    A positions in order (the candidates' global order)."""
    if chunk < 2 or chunk % 2:
        raise ValueError("chunk must be even and >= 2")
    if n_sink < 0 or n_recent < 0 or n_sink + n_recent > n:
        raise ValueError("need 0 <= n_sink, n_recent and n_sink + n_recent <= n")
    lo, hi = n_sink, n - n_recent
    chunks = [(s, min(s + chunk, hi)) for s in range(lo, hi, chunk)]
    a_pos = [p for (s, e) in chunks for p in range(s, e, 2)]
    return chunks, a_pos


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    na = math.sqrt(float(np.dot(a, a)))
    nb = math.sqrt(float(np.dot(b, b)))
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b)) / (na * nb)


def csm_match(k: np.ndarray, chunk: int, n_sink: int, n_recent: int):
    """Best B partner of every A token of one slab (k: [n, d] float64).

    Returns (a_pos [n_A] int64, score [n_A] float64 (-inf without a
    candidate), match [n_A] int64 (the partner's position, -1 without one)).
    """
    n = k.shape[0]
    chunks, a_pos = csm_layout(n, chunk, n_sink, n_recent)
    score = np.full(len(a_pos), -np.inf)
    match = np.full(len(a_pos), -1, dtype=np.int64)
    i = 0
    for (s, e) in chunks:
        b_pos = list(range(s + 1, e, 2))
        for a in range(s, e, 2):
            best, best_b = -np.inf, -1
            for b in b_pos:  # ascending, so a strict > keeps the lower position on ties
                c = cosine(k[a], k[b])
                if c > best:
                    best, best_b = c, b
            score[i], match[i] = best, best_b
            i += 1
    return np.asarray(a_pos, dtype=np.int64), score, match


def csm_select(score: np.ndarray, n_merge: int) -> np.ndarray:
    """Indices (into the A list) of the n_merge candidates with the highest
    similarity, ties to the lower A position; ascending."""
    n_cand = int(np.isfinite(score).sum())
    if not (0 <= n_merge <= n_cand):
        raise ValueError("need 0 <= n_merge <= number of candidates")
    order = np.lexsort((np.arange(score.shape[0]), -score))
    return np.sort(order[:n_merge]).astype(np.int64)


def csm_merge(k: np.ndarray, v: np.ndarray, degree: np.ndarray, a_pos: np.ndarray, match: np.ndarray,
              chosen: np.ndarray):
    """Apply the chosen merges (indices into the A list) to one slab: each
    chosen A token joins its partner's cluster; clusters become degree-weighted
    means. Returns (k_out [n - m, d], v_out, degree_out [n - m], merged [n - m]
    bool: whether the survivor is a centroid of more than one token) with the
    survivors in position order, keys and values in float64."""
    n = k.shape[0]
    removed = np.zeros(n, dtype=bool)
    wk = k * degree[:, None]
    wv = v * degree[:, None]
    deg = degree.astype(np.float64).copy()
    acc_k, acc_v = wk.copy(), wv.copy()
    merged = np.zeros(n, dtype=bool)
    for i in chosen:
        a, b = int(a_pos[i]), int(match[i])
        if b < 0:
            raise ValueError("a chosen token has no candidate")
        removed[a] = True
        acc_k[b] += wk[a]
        acc_v[b] += wv[a]
        deg[b] += degree[a]
        merged[b] = True
    keep = ~removed
    k_out = np.where(merged[:, None], acc_k / deg[:, None], k)[keep]
    v_out = np.where(merged[:, None], acc_v / deg[:, None], v)[keep]
    return k_out, v_out, deg[keep].astype(np.int64), merged[keep]


def csm_round(k: np.ndarray, v: np.ndarray, degree: Optional[np.ndarray], chunk: int, n_sink: int, n_recent: int,
              n_merge: int) -> dict:
    """One CSM round on one slab (k, v: [n, d] float64; degree [n] or None
    for all ones): match, select, merge."""
    degree = np.ones(k.shape[0], dtype=np.int64) if degree is None else np.asarray(degree, dtype=np.int64)
    a_pos, score, match = csm_match(k, chunk, n_sink, n_recent)
    chosen = csm_select(score, n_merge)
    k_out, v_out, deg_out, merged = csm_merge(k, v, degree, a_pos, match, chosen)
    return {"a_pos": a_pos, "score": score, "match": match, "chosen": chosen, "k": k_out, "v": v_out,
            "degree": deg_out, "merged": merged}


def merge_count(rate: float, n: int, n_sink: int, n_recent: int) -> int:
    """Merges of one round at compression ratio ``rate``: floor(rate * middle
    tokens); the progressive schedule lowers the rate linearly over rounds."""
    return int(math.floor(rate * (n - n_sink - n_recent) + 1e-9))


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, degree: Optional[np.ndarray],
                     scale: float) -> np.ndarray:
    """One decode step over a (compacted) cache of one sequence:
    q [Hq, d], k, v [Hkv, n, d] float64, degree [Hkv, n] or None.
    out[h] = sum_j p_j v[g, j] with p = softmax_j(scale * <q_h, k[g, j]> +
    ln degree[g, j]), g = h // (Hq / Hkv)."""
    Hq, d = q.shape
    Hkv, n, _ = k.shape
    G = Hq // Hkv
    out = np.empty((Hq, v.shape[2]))
    for h in range(Hq):
        g = h // G
        logit = scale * (k[g] @ q[h])
        if degree is not None:
            logit = logit + np.log(np.asarray(degree[g], dtype=np.float64))
        m = logit.max()
        p = np.exp(logit - m)
        out[h] = (p @ v[g]) / p.sum()
    return out
