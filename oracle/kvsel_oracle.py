"""fp64 CPU oracle for attention-saliency token selection.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does, and it shares no code with the HIP kernels.

What is computed, and where the pages state it:

* FastKV (page "FastKV: Decoupling of Context Reduction and KV Cache
  Compression ...", section 2A "Token-Selective Propagation"): the TSP layer
  ranks tokens by a saliency score and passes on only the most informative
  tokens plus a window of the newest tokens.
* StructKV (page "StructKV: Preserving the Structural Skeleton ...", section
  1 "Global In-Degree Centrality"): a token's score is its attention scores
  summed over all layers up to the pivot.
* FastKV section 2B and StructKV section 3: the number of tokens propagated
  (TSP rate / compute budget) and the number of KV entries kept
  (KV-retention rate / storage budget) are independent knobs.

The pages give no formula for the saliency score. The reading used here (the
observation-window attention score of SnapKV, which both pages name as prior
art) is, per sequence and layer, with G = Hq / Hkv, query head h using KV head
g = floor(h / G), scale = 1 / sqrt(d), and window query i at position
p_i = N - w + i seeing keys j <= p_i:

    l[h, i, j]  = scale * <q[h, i], k[g, j]>
    lse[h, i]   = log sum_{j <= p_i} exp(l[h, i, j])
    raw[g, j]   = (1 / G) * sum_{h in group g} sum_i exp(l[h, i, j] - lse[h, i])
    s[g, j]     = (1 / kp) * sum_{t = -r..r} raw[g, j + t],  j in [0, N - w),
                  raw taken as 0 outside [0, N - w), r = (kp - 1) / 2
    C[g, j]     = sum over layers of s           (StructKV accumulation)
    T[j]        = (1 / Hkv) * sum_g s[g, j]      (token-set score for TSP)
    keep        = the (budget - w) prefix positions with the largest score,
                  ties to the lower position, plus the window N - w .. N - 1,
                  listed in ascending position
    gathered    = the kept rows of K / V (or hidden states), bit for bit

Every floating-point step runs in float64 on the exact input values (bf16 or
fp32 widened exactly). A matrix product (BLAS) computes the dot products and a
stable sort orders the scores; nothing is blocked, fused or reordered beyond
that.
"""

from __future__ import annotations

import concurrent.futures as cf
import math
from typing import Optional, Sequence

import numpy as np

try:  # keep BLAS single-threaded inside worker threads
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None


# ---------------------------------------------------------------------------
# input widening
# ---------------------------------------------------------------------------
def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) or fp32 values to float64."""
    if dtype == "bf16":
        b = np.ascontiguousarray(x, dtype=np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# one (layer, sequence): window attention, LSE and per-KV-head saliency
# ---------------------------------------------------------------------------
def window_logits(q_h: np.ndarray, k_g: np.ndarray, scale: float) -> np.ndarray:
    """Scaled logits of the w window queries of one head against all N keys,
    with the causal mask applied (-inf where key j > N - w + i).

    q_h: [w, d] float64, k_g: [N, d] float64 -> [w, N] float64.
    """
    w = q_h.shape[0]
    N = k_g.shape[0]
    logits = (q_h @ k_g.T) * scale
    # window query i sits at position N - w + i and may not see later keys
    i = np.arange(w)[:, None]
    j = np.arange(N - w, N)[None, :]
    future = j > (N - w + i)
    logits[:, N - w:][future] = -np.inf
    return logits


def row_lse(logits: np.ndarray) -> np.ndarray:
    """Log-sum-exp of each row, shifted by the row maximum so that exp never
    overflows (logits of +-1000 are fine)."""
    m = logits.max(axis=1, keepdims=True)
    z = np.exp(logits - m).sum(axis=1, keepdims=True)
    return (m + np.log(z))[:, 0]


def _saliency_group(q_grp: np.ndarray, k_g: np.ndarray, scale: float):
    """The G heads of one KV group: (lse [G, w], raw [N]) with the 1/G mean."""
    G = q_grp.shape[0]
    lse = np.empty(q_grp.shape[:2])
    raw = np.zeros(k_g.shape[0])
    for hl in range(G):
        logits = window_logits(q_grp[hl], k_g, scale)
        lse[hl] = row_lse(logits)
        raw += np.exp(logits - lse[hl][:, None]).sum(axis=0)
    return lse, raw / G


def saliency_one(q: np.ndarray, k: np.ndarray, scale: Optional[float] = None):
    """One (layer, sequence).

    q: [Hq, w, d] float64 window queries; k: [Hkv, N, d] float64 keys.
    Returns (lse [Hq, w], raw [Hkv, N]); raw covers all N keys, window keys
    included, so that sum_j raw[g, j] == w for every g.
    """
    Hq, w, d = q.shape
    Hkv, N, _ = k.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    scale = default_scale(d) if scale is None else scale
    lse = np.empty((Hq, w))
    raw = np.empty((Hkv, N))
    for g in range(Hkv):
        lse[g * G:(g + 1) * G], raw[g] = _saliency_group(q[g * G:(g + 1) * G], k[g], scale)
    return lse, raw


def saliency_all(q: np.ndarray, k: np.ndarray, dtype: str, scale: Optional[float] = None,
                 threads: int = 1, heads: Optional[Sequence[int]] = None):
    """Every (layer, sequence, KV group) of a workload.

    q: [L, B, Hq, w, d], k: [L, B, Hkv, N, d] in the stored element type
    (bf16 bits or fp32). ``heads`` restricts the work to some KV heads (the
    others come back as NaN). Independent (layer, sequence, KV head) units run
    on ``threads`` worker threads; each unit is computed exactly as
    ``saliency_one`` would.

    Returns (lse [L, B, Hq, w], raw [L, B, Hkv, N]) float64.
    """
    L, B, Hq, w, d = q.shape
    _, _, Hkv, N, _ = k.shape
    G = Hq // Hkv
    scale = default_scale(d) if scale is None else scale
    heads = list(range(Hkv)) if heads is None else list(heads)
    lse = np.full((L, B, Hq, w), np.nan)
    raw = np.full((L, B, Hkv, N), np.nan)

    def unit(args):
        l, b, g = args
        qg = to_f64(q[l, b, g * G:(g + 1) * G], dtype)
        kg = to_f64(k[l, b, g], dtype)
        lse_g, raw_g = _saliency_group(qg, kg, scale)
        lse[l, b, g * G:(g + 1) * G] = lse_g
        raw[l, b, g] = raw_g

    jobs = [(l, b, g) for l in range(L) for b in range(B) for g in heads]
    if threads <= 1:
        for j in jobs:
            unit(j)
    else:
        ctx = threadpool_limits(1) if threadpool_limits is not None else _null()
        with ctx, cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(unit, jobs))
    return lse, raw


def saliency_given_lse(q: np.ndarray, k: np.ndarray, lse: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """One (layer, sequence) with the window rows' natural-log LSE handed in:
    prefill attention has already normalised every window row (FastKV section
    2A, StructKV section 1), so each key's score needs only its logits and the
    given LSE: raw[g, j] = (1/G) sum over the G heads h of group g and the w
    rows i of exp(l[h, i, j] - lse[h, i]), over the keys row i sees.

    q: [Hq, w, d], k: [Hkv, N, d], lse: [Hq, w] float64 -> raw [Hkv, N].
    """
    Hq, w, d = q.shape
    Hkv, N, _ = k.shape
    G = Hq // Hkv
    scale = default_scale(d) if scale is None else scale
    raw = np.zeros((Hkv, N))
    for h in range(Hq):
        logits = window_logits(q[h], k[h // G], scale)
        raw[h // G] += np.exp(logits - lse[h][:, None]).sum(axis=0)
    return raw / G


def saliency_all_given_lse(q: np.ndarray, k: np.ndarray, lse: np.ndarray, dtype: str,
                           scale: Optional[float] = None, threads: int = 1) -> np.ndarray:
    """saliency_given_lse over every (layer, sequence): q [L, B, Hq, w, d],
    k [L, B, Hkv, N, d] (stored element type), lse [L, B, Hq, w] -> raw
    [L, B, Hkv, N] float64."""
    L, B = q.shape[:2]
    raw = np.full((L, B, k.shape[2], k.shape[3]), np.nan)

    def unit(args):
        l, b = args
        raw[l, b] = saliency_given_lse(to_f64(q[l, b], dtype), to_f64(k[l, b], dtype),
                                       np.asarray(lse[l, b], dtype=np.float64), scale)

    jobs = [(l, b) for l in range(L) for b in range(B)]
    if threads <= 1:
        for j in jobs:
            unit(j)
    else:
        ctx = threadpool_limits(1) if threadpool_limits is not None else _null()
        with ctx, cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(unit, jobs))
    return raw


class _null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


# ---------------------------------------------------------------------------
# pivot statistics (StructKV section 2, dynamic pivot detection)
# ---------------------------------------------------------------------------
def row_stats(q: np.ndarray, k: np.ndarray, small_p: float, scale: Optional[float] = None):
    """Attention statistics of every window row of one (layer, sequence).

    StructKV section 2 watches attention entropy, sparsity and variance during
    the first pass and looks for the layer where entropy falls and sparsity
    rises. Row i of head h has the distribution p_j = exp(l_j - LSE) over the
    keys it sees (j <= N - w + i, n_i = N - w + i + 1 of them):

        entropy = -sum_j p_j ln p_j                  (nats)
        sum_p2  = sum_j p_j^2                        (the row's variance is
                                                      sum_p2 / n_i - 1 / n_i^2)
        n_below = number of visible j with p_j < small_p   (sparsity = n_below / n_i)

    q: [Hq, w, d], k: [Hkv, N, d] float64. Returns (entropy [Hq, w],
    sum_p2 [Hq, w], n_below [Hq, w] int64).
    """
    Hq, w, d = q.shape
    Hkv, N, _ = k.shape
    G = Hq // Hkv
    scale = default_scale(d) if scale is None else scale
    entropy = np.empty((Hq, w))
    sum_p2 = np.empty((Hq, w))
    n_below = np.empty((Hq, w), dtype=np.int64)
    for h in range(Hq):
        g = h // G  # the KV head this query head reads
        logits = window_logits(q[h], k[g], scale)
        visible = np.isfinite(logits)
        logp = np.where(visible, logits - row_lse(logits)[:, None], 0.0)
        p = np.where(visible, np.exp(logp), 0.0)
        entropy[h] = -(p * logp).sum(axis=1)
        sum_p2[h] = (p * p).sum(axis=1)
        n_below[h] = (visible & (p < small_p)).sum(axis=1)
    return entropy, sum_p2, n_below


def row_stats_all(q: np.ndarray, k: np.ndarray, dtype: str, small_p: float, scale: Optional[float] = None,
                  threads: int = 1):
    """row_stats over every (layer, sequence): q [L, B, Hq, w, d], k [L, B, Hkv,
    N, d] in the stored element type -> (entropy, sum_p2, n_below), each
    [L, B, Hq, w]."""
    L, B, Hq, w, _ = q.shape
    ent = np.full((L, B, Hq, w), np.nan)
    sp2 = np.full((L, B, Hq, w), np.nan)
    nb = np.zeros((L, B, Hq, w), dtype=np.int64)

    def unit(args):
        l, b = args
        ent[l, b], sp2[l, b], nb[l, b] = row_stats(to_f64(q[l, b], dtype), to_f64(k[l, b], dtype), small_p, scale)

    jobs = [(l, b) for l in range(L) for b in range(B)]
    if threads <= 1:
        for j in jobs:
            unit(j)
    else:
        ctx = threadpool_limits(1) if threadpool_limits is not None else _null()
        with ctx, cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(unit, jobs))
    return ent, sp2, nb


def layer_summary(entropy: np.ndarray, sum_p2: np.ndarray, n_below: np.ndarray, n_keys: int):
    """Per-layer means over (sequence, head, window row) of the row entropy,
    the sparsity n_below / n_i and the variance sum_p2 / n_i - 1 / n_i^2.
    Inputs [L, B, Hq, w]; returns three [L] arrays."""
    w = entropy.shape[-1]
    n = (n_keys - w + 1 + np.arange(w)).astype(np.float64)  # keys row i sees
    ent = entropy.reshape(entropy.shape[0], -1, w)
    spars = (n_below / n).reshape(ent.shape)
    var = (sum_p2 / n - 1.0 / (n * n)).reshape(ent.shape)
    return ent.mean(axis=(1, 2)), spars.mean(axis=(1, 2)), var.mean(axis=(1, 2))


def pivot_layer(mean_entropy: Sequence[float], mean_sparsity: Sequence[float], min_drop: float,
                min_rise: float) -> int:
    """StructKV's pivot: the first layer l >= 1 at which the attention pattern
    changes phase, read as the mean entropy falling by at least ``min_drop``
    (a fraction of layer l-1's entropy) while the mean sparsity rises by at
    least ``min_rise`` (an absolute fraction), both against layer l-1. Layers
    0 .. pivot are accumulated. Without such a layer the pivot is the last
    layer."""
    L = len(mean_entropy)
    if L < 1 or len(mean_sparsity) != L:
        raise ValueError("need one entropy and one sparsity value per layer")
    for l in range(1, L):
        fell = mean_entropy[l - 1] - mean_entropy[l] >= min_drop * mean_entropy[l - 1]
        rose = mean_sparsity[l] - mean_sparsity[l - 1] >= min_rise
        if fell and rose:
            return l
    return L - 1


# ---------------------------------------------------------------------------
# pool, accumulate
# ---------------------------------------------------------------------------
def avg_pool(raw_prefix: np.ndarray, kernel: int) -> np.ndarray:
    """Stride-1, same-length average pool over the last axis with zero padding
    of r = (kernel - 1) / 2 on each side; the divisor is always ``kernel``."""
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and >= 1")
    r = (kernel - 1) // 2
    n = raw_prefix.shape[-1]
    padded = np.zeros(raw_prefix.shape[:-1] + (n + 2 * r,))
    padded[..., r:r + n] = raw_prefix
    out = np.zeros(raw_prefix.shape)
    for t in range(kernel):
        out += padded[..., t:t + n]
    return out / kernel


def max_pool(raw_prefix: np.ndarray, kernel: int) -> np.ndarray:
    """Stride-1, same-length max pool over the last axis: position j takes the
    largest value among positions j - r .. j + r that lie inside the row
    (r = (kernel - 1) / 2). Raw scores are >= 0, so this equals zero padding."""
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and >= 1")
    r = (kernel - 1) // 2
    n = raw_prefix.shape[-1]
    padded = np.full(raw_prefix.shape[:-1] + (n + 2 * r,), -np.inf)
    padded[..., r:r + n] = raw_prefix
    out = np.full(raw_prefix.shape, -np.inf)
    for tap in range(kernel):
        out = np.maximum(out, padded[..., tap:tap + n])
    return out


def pooled_scores(raw: np.ndarray, window: int, kernel: int, pool_type: str = "avg") -> np.ndarray:
    """Ranked score of the prefix keys: the pool of raw[..., :N - w] (average,
    or with ``pool_type="max"`` the max-pool variant); the window keys are
    always kept and are neither ranked nor pooled."""
    N = raw.shape[-1]
    if pool_type == "max":
        return max_pool(raw[..., :N - window], kernel)
    return avg_pool(raw[..., :N - window], kernel)


def accumulate_layers(per_layer: np.ndarray) -> np.ndarray:
    """StructKV global centrality: the layer scores added up over the layer
    axis (axis 0), in layer order."""
    acc = np.zeros(per_layer.shape[1:])
    for s in per_layer:
        acc = acc + s
    return acc


def head_mean(s: np.ndarray) -> np.ndarray:
    """Token-set score for TSP: mean over the KV-head axis (axis -2), keeping
    it as a length-1 axis: [..., H, n] -> [..., 1, n]."""
    return s.mean(axis=-2, keepdims=True)


# ---------------------------------------------------------------------------
# select
# ---------------------------------------------------------------------------
def select_row(score: np.ndarray, n_keys: int, window: int, budget: int, n_sink: int = 0) -> np.ndarray:
    """Kept positions of one selection row.

    score: [N - w] prefix scores. The (budget - w) positions with the largest
    score are kept, a tie going to the lower position, then the window
    N - w .. N - 1 is added; the result is sorted ascending (int64, length
    ``budget``). With ``n_sink`` > 0 the attention sinks 0 .. n_sink-1 are
    always kept (CentroidKV section 2 preserves sinks and recent tokens) and
    take n_sink of the (budget - w) slots.
    """
    n_prefix = n_keys - window
    if score.shape[-1] != n_prefix:
        raise ValueError("score length must be N - w")
    if not (window <= budget <= n_keys):
        raise ValueError("need window <= budget <= N")
    kk = budget - window
    if not (0 <= n_sink <= kk):
        raise ValueError("need 0 <= n_sink <= budget - window")
    pos = np.arange(n_prefix)
    order = np.lexsort((pos, -np.asarray(score, dtype=np.float64)))  # score desc, position asc
    if n_sink:
        order = np.concatenate([pos[:n_sink], order[order >= n_sink]])  # sinks first
    kept = np.concatenate([np.sort(order[:kk]), np.arange(n_prefix, n_keys)])
    return kept.astype(np.int64)


def select(scores: np.ndarray, n_keys: int, window: int, budget: int, n_sink: int = 0) -> np.ndarray:
    """select_row over every leading index: [..., N - w] -> [..., budget]."""
    lead = scores.shape[:-1]
    flat = scores.reshape(-1, scores.shape[-1])
    out = np.stack([select_row(r, n_keys, window, budget, n_sink) for r in flat]) if flat.shape[0] else \
        np.zeros((0, budget), dtype=np.int64)
    return out.reshape(lead + (budget,))


# ---------------------------------------------------------------------------
# gather
# ---------------------------------------------------------------------------
def gather_rows(src: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Copy the kept rows: out[..., t, :] = src[..., idx[..., t], :].

    src: [P, N, row] (any element type, copied bit for bit); idx: [P or 1, budget].
    """
    P = src.shape[0]
    out = np.empty((P, idx.shape[-1]) + src.shape[2:], dtype=src.dtype)
    for p in range(P):
        out[p] = src[p][idx[p if idx.shape[0] > 1 else 0]]
    return out


# ---------------------------------------------------------------------------
# the whole path for one workload
# ---------------------------------------------------------------------------
def pipeline(q: np.ndarray, k: np.ndarray, v: Optional[np.ndarray], *, dtype: str, window: int,
             pool_kernel: int, kv_budget: int, tsp_budget: Optional[int] = None,
             hidden: Optional[np.ndarray] = None, scale: Optional[float] = None,
             threads: int = 1, heads: Optional[Sequence[int]] = None,
             lse_in: Optional[np.ndarray] = None, pool_type: str = "avg", n_sink: int = 0) -> dict:
    """Score every layer, accumulate over layers (StructKV; a single layer is
    its own sum), select per KV head with the KV budget, and gather K and V of
    every layer with those indices; with a TSP budget also rank the head-mean
    score for one token set per sequence and gather the hidden rows. With
    ``lse_in`` ([L, B, Hq, w] natural-log LSE of the window rows, handed in)
    the scores use that LSE instead of computing it. ``pool_type`` = "max"
    takes the max-pool variant; ``n_sink`` protects the first positions in
    both selections.

    Shapes: q [L, B, Hq, w, d]; k, v [L, B, Hkv, N, d]; hidden [B, N, D].
    """
    L, B, Hq, w, d = q.shape
    N = k.shape[3]
    Hkv = k.shape[2]
    if lse_in is None:
        lse, raw = saliency_all(q, k, dtype, scale, threads=threads, heads=heads)
    else:
        lse = np.asarray(lse_in, dtype=np.float64)
        raw = saliency_all_given_lse(q, k, lse, dtype, scale, threads=threads)
    per_layer = pooled_scores(raw, window, pool_kernel, pool_type)  # [L, B, Hkv, Np]
    scores = accumulate_layers(per_layer)                         # [B, Hkv, Np]
    hsel = list(range(Hkv)) if heads is None else list(heads)
    idx = np.zeros((B, Hkv, kv_budget), dtype=np.int64)
    for b in range(B):
        for g in hsel:
            idx[b, g] = select_row(scores[b, g], N, window, kv_budget, n_sink)
    out = {"lse": lse, "raw": raw, "scores": scores, "idx": idx}
    if v is not None:
        kc = np.empty((L, B, Hkv, kv_budget, d), dtype=k.dtype)
        vc = np.empty_like(kc)
        for l in range(L):
            for b in range(B):
                kc[l, b] = gather_rows(k[l, b], idx[b])
                vc[l, b] = gather_rows(v[l, b], idx[b])
        out["k_kept"], out["v_kept"] = kc, vc
    if tsp_budget is not None:
        tscore = head_mean(scores)                               # [B, 1, Np]
        tidx = select(tscore, N, window, tsp_budget, n_sink)     # [B, 1, budget]
        out["tsp_scores"], out["tsp_idx"] = tscore, tidx
        if hidden is not None:
            out["hidden_kept"] = np.stack([hidden[b][tidx[b, 0]] for b in range(B)])
    return out
