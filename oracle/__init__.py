"""fp64 CPU oracle (test infrastructure only; see kvsel_oracle)."""

from .kvsel_oracle import (
    to_f64,
    default_scale,
    window_logits,
    row_lse,
    saliency_one,
    saliency_all,
    saliency_given_lse,
    saliency_all_given_lse,
    avg_pool,
    pooled_scores,
    accumulate_layers,
    head_mean,
    select_row,
    select,
    gather_rows,
    pipeline,
)

__all__ = [
    "to_f64",
    "default_scale",
    "window_logits",
    "row_lse",
    "saliency_one",
    "saliency_all",
    "saliency_given_lse",
    "saliency_all_given_lse",
    "avg_pool",
    "pooled_scores",
    "accumulate_layers",
    "head_mean",
    "select_row",
    "select",
    "gather_rows",
    "pipeline",
]
