"""Seeded synthetic inputs for attention-saliency token selection.

This package holds the workload table (shapes, budgets, value distributions)
and the seeded generators that turn a workload into Q / K / V / hidden-state
arrays. It holds none of the selection method's arithmetic: both the fp64
oracle and the HIP path read the arrays it produces, and nothing else is
shared between them.
"""

from .configs import Workload, WORKLOADS, get_workload, budget_from_rate
from .gen import make_inputs, bf16_bits_to_f32, f64_to_bf16_bits, layer_seed

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "budget_from_rate",
    "make_inputs",
    "bf16_bits_to_f32",
    "f64_to_bf16_bits",
    "layer_seed",
]
