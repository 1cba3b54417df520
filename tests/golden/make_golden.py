"""Write oracle_regression.json: the fp64 oracle's outputs on small seeded
inputs (a regression record of the oracle itself; see README.md). Calls only
the oracle."""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def inputs():
    rng = np.random.default_rng(2024)
    q = rng.normal(size=(2, 1, 4, 3, 8)).astype(np.float32)   # [L, B, Hq, w, d]
    k = rng.normal(size=(2, 1, 2, 40, 8)).astype(np.float32)  # [L, B, Hkv, N, d]
    k[:, :, :, 7] *= 3.0  # one hub
    v = rng.normal(size=(2, 1, 2, 40, 8)).astype(np.float32)
    return q, k, v


def compute():
    q, k, v = inputs()
    out = {}
    ref = oracle.pipeline(q, k, v, dtype="f32", window=3, pool_kernel=3, kv_budget=12, tsp_budget=15)
    out["lse"] = ref["lse"].tolist()
    out["scores"] = ref["scores"].tolist()
    out["idx"] = ref["idx"].tolist()
    out["tsp_idx"] = ref["tsp_idx"].tolist()
    mx = oracle.pipeline(q, k, None, dtype="f32", window=3, pool_kernel=3, kv_budget=12, pool_type="max", n_sink=2)
    out["max_pool_scores"] = mx["scores"].tolist()
    out["sink_idx"] = mx["idx"].tolist()
    ent, sp2, nb = oracle.row_stats_all(q, k, "f32", 0.02)
    out["entropy"] = ent.tolist()
    out["sum_p2"] = sp2.tolist()
    out["n_below"] = nb.tolist()
    k64 = oracle.to_f64(k[0, 0, 0], "f32")
    v64 = oracle.to_f64(v[0, 0, 0], "f32")
    r = oracle.csm_round(k64, v64, None, 4, 2, 3, 6)
    out["csm_k"] = r["k"].tolist()
    out["csm_degree"] = r["degree"].tolist()
    out["csm_chosen"] = r["chosen"].tolist()
    out["decode"] = oracle.decode_attention(oracle.to_f64(q[0, 0, :, 0], "f32"), oracle.to_f64(k[0, 0], "f32"),
                                            oracle.to_f64(v[0, 0], "f32"), None, 0.35).tolist()
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(compute(), f)
    print("wrote", os.path.join(HERE, "oracle_regression.json"))
