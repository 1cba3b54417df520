"""Each pin set must catch a plausible mistake planted in a copy of the
oracle (on the CPU): a dropped term, a wrong sign or index, a transposed
operand, a wrong divisor, a reversed tie-break."""

import os
import types

import pytest

import centroid_checks
import oracle_checks

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "kvsel_oracle.py")
CENTROID_SRC = os.path.join(ORACLE_DIR, "centroid_oracle.py")

MUTATIONS = {
    "no_causal_mask": ("future = j > (N - w + i)", "future = j > N"),
    "causal_off_by_one": ("future = j > (N - w + i)", "future = j >= (N - w + i)"),
    "no_max_shift": ("z = np.exp(logits - m).sum(axis=1, keepdims=True)\n    return (m + np.log(z))[:, 0]",
                     "z = np.exp(logits).sum(axis=1, keepdims=True)\n    return np.log(z)[:, 0]"),
    "lse_sign": ("raw += np.exp(logits - lse[hl][:, None]).sum(axis=0)",
                 "raw += np.exp(logits + lse[hl][:, None]).sum(axis=0)"),
    "no_gqa_mean": ("return lse, raw / G", "return lse, raw"),
    "gqa_interleaved": ("_saliency_group(q[g * G:(g + 1) * G], k[g], scale)",
                        "_saliency_group(q[g::Hkv], k[g], scale)"),
    "scale_wrong": ("return 1.0 / math.sqrt(head_dim)", "return 1.0 / head_dim"),
    "transposed_keys": ("logits = (q_h @ k_g.T) * scale", "logits = (q_h @ k_g[::-1].T) * scale"),
    "pool_divisor": ("return out / kernel", "return out / max(1, kernel - 1)"),
    "pool_dropped_tap": ("for t in range(kernel):", "for t in range(kernel - 1):"),
    "pool_over_window": ("return avg_pool(raw[..., :N - window], kernel)",
                         "return avg_pool(raw, kernel)[..., :N - window]"),
    "tie_break_reversed": ("order = np.lexsort((pos, -np.asarray(score, dtype=np.float64)))",
                           "order = np.lexsort((-pos, -np.asarray(score, dtype=np.float64)))"),
    "ascending_scores": ("order = np.lexsort((pos, -np.asarray(score, dtype=np.float64)))",
                         "order = np.lexsort((pos, np.asarray(score, dtype=np.float64)))"),
    "window_not_kept": ("kept = np.concatenate([np.sort(order[:kk]), np.arange(n_prefix, n_keys)])",
                        "kept = np.sort(order[:budget])"),
    "layer_dropped": ("acc = acc + s", "acc = s"),
    "head_sum": ("return s.mean(axis=-2, keepdims=True)", "return s.sum(axis=-2, keepdims=True)"),
    "gather_off_by_one": ("out[p] = src[p][idx[p if idx.shape[0] > 1 else 0]]",
                          "out[p] = src[p][np.minimum(idx[p if idx.shape[0] > 1 else 0] + 1, src.shape[1] - 1)]"),
    "bf16_widening": ("(b.astype(np.uint32) << 16)", "(b.astype(np.uint32) << 15)"),
    "max_pool_dropped_tap": ("for tap in range(kernel):", "for tap in range(kernel - 1):"),
    "max_pool_as_avg": ("        return max_pool(raw[..., :N - window], kernel)", "        return avg_pool(raw[..., :N - window], kernel)"),
    "sinks_dropped": ("        order = np.concatenate([pos[:n_sink], order[order >= n_sink]])  # sinks first", "        pass"),
    "sinks_off_by_one": ("        order = np.concatenate([pos[:n_sink], order[order >= n_sink]])  # sinks first",
                         "        order = np.concatenate([pos[:n_sink - 1], order[order >= n_sink - 1]])"),
    "stats_wrong_group": ("        g = h // G  # the KV head this query head reads", "        g = h % Hkv"),
    "stats_entropy_sign": ("        entropy[h] = -(p * logp).sum(axis=1)", "        entropy[h] = (p * logp).sum(axis=1)"),
    "stats_p2_unsquared": ("        sum_p2[h] = (p * p).sum(axis=1)", "        sum_p2[h] = p.sum(axis=1)"),
    "stats_count_masked": ("        n_below[h] = (visible & (p < small_p)).sum(axis=1)", "        n_below[h] = (p < small_p).sum(axis=1)"),
    "stats_count_above": ("        n_below[h] = (visible & (p < small_p)).sum(axis=1)", "        n_below[h] = (visible & (p > small_p)).sum(axis=1)"),
    "summary_n_off_by_one": ("    n = (n_keys - w + 1 + np.arange(w)).astype(np.float64)", "    n = (n_keys - w + np.arange(w)).astype(np.float64)"),
    "pivot_off_by_one": ("            return l\n    return L - 1", "            return l - 1\n    return L - 1"),
    "pivot_fall_or_rise": ("        if fell and rose:", "        if fell or rose:"),
    "pivot_absolute_drop": ("        fell = mean_entropy[l - 1] - mean_entropy[l] >= min_drop * mean_entropy[l - 1]",
                            "        fell = mean_entropy[l - 1] - mean_entropy[l] >= min_drop"),
    "given_lse_sign": ("raw[h // G] += np.exp(logits - lse[h][:, None]).sum(axis=0)",
                       "raw[h // G] += np.exp(logits + lse[h][:, None]).sum(axis=0)"),
    "given_lse_no_mean": ("    return raw / G\n\n\ndef saliency_all_given_lse", "    return raw\n\n\ndef saliency_all_given_lse"),
    "given_lse_wrong_group": ("logits = window_logits(q[h], k[h // G], scale)", "logits = window_logits(q[h], k[h % Hkv], scale)"),
    "given_lse_all_lse_swapped": ("np.asarray(lse[l, b], dtype=np.float64), scale)",
                                  "np.asarray(lse[b, l], dtype=np.float64), scale)"),
    "given_lse_all_wrong_slice": ("raw[l, b] = saliency_given_lse(to_f64(q[l, b], dtype), to_f64(k[l, b], dtype),",
                                  "raw[l, b] = saliency_given_lse(to_f64(q[l, b], dtype), to_f64(k[l, 0], dtype),"),
    "given_lse_all_out_swapped": ("        raw[l, b] = saliency_given_lse(", "        raw[b, l] = saliency_given_lse("),
    "stats_all_wrong_slice": ("row_stats(to_f64(q[l, b], dtype), to_f64(k[l, b], dtype), small_p, scale)",
                              "row_stats(to_f64(q[l, b], dtype), to_f64(k[b, l], dtype), small_p, scale)"),
    "stats_all_out_swapped": ("        ent[l, b], sp2[l, b], nb[l, b] = row_stats(",
                              "        ent[b, l], sp2[b, l], nb[b, l] = row_stats("),
    "stats_all_first_seq_only": ("    jobs = [(l, b) for l in range(L) for b in range(B)]\n    if threads <= 1:\n        for j in jobs:\n            unit(j)\n    else:\n        ctx = threadpool_limits(1) if threadpool_limits is not None else _null()\n        with ctx, cf.ThreadPoolExecutor(threads) as ex:\n            list(ex.map(unit, jobs))\n    return ent, sp2, nb",
                                 "    jobs = [(l, b) for l in range(L) for b in range(1)]\n    if threads <= 1:\n        for j in jobs:\n            unit(j)\n    else:\n        ctx = threadpool_limits(1) if threadpool_limits is not None else _null()\n        with ctx, cf.ThreadPoolExecutor(threads) as ex:\n            list(ex.map(unit, jobs))\n    return ent, sp2, nb"),
}


CENTROID_MUTATIONS = {
    "csm_partition_swapped": ("    a_pos = [p for (s, e) in chunks for p in range(s, e, 2)]",
                              "    a_pos = [p for (s, e) in chunks for p in range(s + 1, e, 2)]"),
    "csm_chunks_from_zero": ("    chunks = [(s, min(s + chunk, hi)) for s in range(lo, hi, chunk)]",
                             "    chunks = [(max(s, lo), min(s + chunk, hi)) for s in range(0, hi, chunk)]"),
    "csm_tie_to_higher_b": ("                if c > best:", "                if c >= best:"),
    "csm_dot_not_cosine": ("    return float(np.dot(a, b)) / (na * nb)", "    return float(np.dot(a, b))"),
    "csm_select_ties_high": ("    order = np.lexsort((np.arange(score.shape[0]), -score))",
                             "    order = np.lexsort((-np.arange(score.shape[0]), -score))"),
    "csm_unweighted_mean": ("    wk = k * degree[:, None]", "    wk = k * 1.0"),
    "csm_degree_not_summed": ("        deg[b] += degree[a]", "        deg[b] += 1"),
    "csm_recent_in_middle": ("    lo, hi = n_sink, n - n_recent", "    lo, hi = n_sink, n"),
    "attn_no_log_degree": ("            logit = logit + np.log(np.asarray(degree[g], dtype=np.float64))", "            pass"),
    "attn_log_sign": ("            logit = logit + np.log(np.asarray(degree[g], dtype=np.float64))",
                      "            logit = logit - np.log(np.asarray(degree[g], dtype=np.float64))"),
    "attn_wrong_group": ("        g = h // G\n        logit", "        g = h % Hkv\n        logit"),
}


def _mutant(old, new, src=SRC):
    text = open(src).read()
    assert text.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("kvsel_oracle_mutant")
    exec(compile(text.replace(old, new), "kvsel_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTATIONS[name])
    failed = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # AssertionError, or the mutant blowing up
            failed.append(check.__name__)
    assert failed, f"no pin caught mutation {name}"


@pytest.mark.parametrize("name", sorted(CENTROID_MUTATIONS))
def test_centroid_pins_catch_planted_mistake(name):
    mod = _mutant(*CENTROID_MUTATIONS[name], src=CENTROID_SRC)
    failed = []
    for check in centroid_checks.CENTROID_CHECKS:
        try:
            check(mod)
        except Exception:
            failed.append(check.__name__)
    assert failed, f"no pin caught mutation {name}"
