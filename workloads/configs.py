"""Workload table: the five synthetic workloads the selection path is built for.

Shapes follow the model families the pages evaluate on (FastKV §4 results:
LLaMA-3.1-8B / Ministral-8B up to 128K tokens; StructKV results: LLaMA-3.1-8B,
Mistral-8B, Qwen-2.5; CentroidKV observations: keys are locally similar along
the sequence). Value distributions are synthetic stand-ins for the
LongBench / RULER / NIAH inputs the pages measure on: no item of those suites
is used.

Budgets count the kept positions *including* the recent window (FastKV §2A:
the selected tokens plus a window of the newest tokens are passed on; the
budget is the total number kept).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple


def budget_from_rate(rate: float, n_keys: int, window: int) -> int:
    """Turn a retention rate (FastKV §2B: TSP rate / KV-retention rate) into a
    kept count: ceil(rate * N), clamped to [window, N]."""
    b = int(math.ceil(rate * n_keys - 1e-9))
    return max(window, min(n_keys, b))


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed namespace of this workload
    dtype: str               # "f32" or "bf16" (Q and K; V / hidden are copied bit-exact)
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_keys: int              # N cached keys per sequence
    window: int              # w: observation window = last w queries, always kept
    pool_kernel: int         # odd avg-pool width (1 = no pool)
    kv_budget: int           # kept per KV head, including the window
    tsp_budget: Optional[int] = None   # token-set budget (TSP), including the window
    rope_base: Optional[float] = None  # rotate-half RoPE base, None = no RoPE
    key_model: str = "gauss"           # "gauss" | "ar1" | "const"
    ar_rho: float = 0.9
    hub_mode: Optional[str] = None     # None | "mean_query" | "norm"
    n_hubs: int = 0
    hub_scale: float = 1.0
    hub_layers: Optional[int] = None   # number of layers (seeded pick) where hubs are active
    sink: bool = False                 # position 0 becomes an attention sink
    sink_scale: float = 6.0
    hidden_dim: Optional[int] = None   # hidden-state width gathered by the token set
    query_model: str = "gauss"         # "gauss" | "zero"
    k_mult: float = 1.0                # extra multiplier on every key (stability cases)
    layer_k_mult: Optional[Tuple[float, ...]] = None  # per-layer key multiplier (sharper attention where larger)

    # derived sizes -------------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_prefix(self) -> int:
        return self.n_keys - self.window

    @property
    def rows(self) -> int:
        """Query rows that score one KV head: G heads x w window queries."""
        return self.group * self.window

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def units(self) -> int:
        """(layer, sequence, KV head, key) units taken through the path."""
        return self.n_layers * self.batch * self.n_kv_heads * self.n_keys

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def compulsory_bytes(self) -> dict:
        """Bytes the path must move at least once (K read once, Q read, final
        scores written and read by the select, indices written, K and V rows
        gathered: read + write; token-set score and hidden rows when a TSP
        budget is set)."""
        L, B, Hq, Hkv, d, N, w = (self.n_layers, self.batch, self.n_q_heads,
                                  self.n_kv_heads, self.head_dim, self.n_keys, self.window)
        e = self.elem_bytes
        Np = N - w
        out = {
            "k_read": L * B * Hkv * N * d * e,
            "q_read": L * B * Hq * w * d * e,
            "scores_rw": 2 * B * Hkv * Np * 4,
            "idx_write": B * Hkv * self.kv_budget * 4,
            "kv_gather": L * 4 * B * Hkv * self.kv_budget * d * e,
        }
        if self.tsp_budget is not None:
            out["tsp_score_rw"] = 2 * B * Np * 4 + B * Hkv * Np * 4
            out["tsp_idx_write"] = B * self.tsp_budget * 4
            if self.hidden_dim:
                out["hidden_gather"] = 2 * B * self.tsp_budget * self.hidden_dim * 2
        out["total"] = sum(out.values())
        return out


# The five workloads. Readings of under-specified details (hub construction,
# sink, AR(1), RoPE convention) are listed with the input recipe in the design
# notes; they change which keys win, never whether two implementations agree.
TINY = Workload(
    name="tiny_f32_2k", wid=1, dtype="f32", n_layers=1, batch=1,
    n_q_heads=8, n_kv_heads=2, head_dim=64, n_keys=2048, window=32,
    pool_kernel=7, kv_budget=256,
    hub_mode="mean_query", n_hubs=16, hub_scale=4.0,
)

LLAMA_32K_TSP = Workload(
    name="llama8b_32k_tsp", wid=2, dtype="bf16", n_layers=1, batch=1,
    n_q_heads=32, n_kv_heads=8, head_dim=128, n_keys=32768, window=8,
    pool_kernel=7, kv_budget=1024, tsp_budget=2048, rope_base=500000.0,
    hub_mode="norm", n_hubs=328, hub_scale=3.0, sink=True, hidden_dim=4096,
)

STRUCTKV_128K = Workload(
    name="structkv_128k_16l", wid=3, dtype="bf16", n_layers=16, batch=1,
    n_q_heads=32, n_kv_heads=8, head_dim=128, n_keys=131072, window=32,
    pool_kernel=7, kv_budget=4096,
    hub_mode="norm", n_hubs=1311, hub_scale=3.0, hub_layers=5,
)

BATCHED_32K_AR1 = Workload(
    name="batched_8x32k_ar1", wid=4, dtype="bf16", n_layers=1, batch=8,
    n_q_heads=32, n_kv_heads=8, head_dim=128, n_keys=32768, window=32,
    pool_kernel=7, kv_budget=budget_from_rate(0.10, 32768, 32),
    key_model="ar1", ar_rho=0.9,
)

QWEN_512K = Workload(
    name="qwen7b_512k", wid=5, dtype="bf16", n_layers=1, batch=1,
    n_q_heads=28, n_kv_heads=4, head_dim=128, n_keys=524288, window=64,
    pool_kernel=7, kv_budget=8192, rope_base=1.0e6,
    hub_mode="norm", n_hubs=524, hub_scale=3.0,
)

WORKLOADS = {w.name: w for w in (TINY, LLAMA_32K_TSP, STRUCTKV_128K, BATCHED_32K_AR1, QWEN_512K)}
WORKLOADS_BY_ID = {w.wid: w for w in WORKLOADS.values()}


def get_workload(key) -> Workload:
    if isinstance(key, int):
        return WORKLOADS_BY_ID[key]
    return WORKLOADS[key]
