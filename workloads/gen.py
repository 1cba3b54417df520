"""Seeded generators for the synthetic workloads.

Recipe (everything drawn from ``numpy.random.default_rng`` seeded with a
``SeedSequence`` whose entropy is ``[workload id, user seed, layer, tensor id,
...]``; tensor ids: 0 = Q, 1 = K, 2 = V, 3 = hub / layer picks, 4 = hidden):

* Q ~ N(0, 1) in fp64 (or all zeros for ``query_model="zero"``), shape
  ``[L, B, Hq, w, d]``; window query i sits at position ``N - w + i``.
* K ~ N(0, 1) in fp64 (``key_model="gauss"``), a stationary AR(1) along the
  sequence ``k_t = rho k_{t-1} + sqrt(1 - rho^2) e_t`` (``"ar1"``, the locally
  similar keys CentroidKV observes), or one random vector repeated at every
  position (``"const"``, used for exact-tie cases). Keys are drawn in blocks of
  ``KEY_BLOCK`` positions, each block with its own seed (AR(1) carries its
  state across blocks).
* ``k_mult`` scales every key; ``layer_k_mult[l]`` scales the keys of layer l
  (larger keys spread the logits, so that layer's attention is sharper: lower
  entropy, more near-zero weights).
* RoPE (rotate-half convention, theta_i = base^(-2i/d)) is applied in fp64 to
  Q and K at their positions when the workload names a base.
* Hubs: ``n_hubs`` positions drawn once per workload from [1, N - w), shared
  by every layer, sequence and KV head. ``"mean_query"`` hubs become
  ``hub_scale * |k_j| * u_g`` with u_g the unit mean of KV group g's post-RoPE
  window queries; ``"norm"`` hubs are scaled by ``hub_scale``. With
  ``hub_layers`` set, hubs are active only in that many seeded layers.
* Sink: position 0 becomes ``sink_scale * sqrt(d) * u_g``.
* Rounding: fp64 -> fp32 -> bf16, both steps round-to-nearest-even.
* V and hidden states are uniformly random finite bit patterns of the element
  type: they are only ever copied, so every bit pattern is a better test of a
  bit-exact copy than a smooth distribution.

None of this is the selection method: it only builds the arrays that both the
oracle and the GPU path read.
"""

from __future__ import annotations

import concurrent.futures as cf
import math
import os
from typing import Iterable, Optional

import numpy as np

from .configs import Workload

KEY_BLOCK = 65536  # positions per independently seeded key block


def layer_seed(wl: Workload, seed: int, layer: int, tensor_id: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.wid, seed, layer, tensor_id, *extra]))


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round to bf16 (via fp32), nearest-even at each step; returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def _round(wl: Workload, x: np.ndarray) -> np.ndarray:
    if wl.dtype == "bf16":
        return f64_to_bf16_bits(x)
    return x.astype(np.float32)


def _rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-(np.arange(half, dtype=np.float64) * 2.0) / d)
    ang = positions.astype(np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _random_finite_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        bad = (b & 0x7F80) == 0x7F80
        b[bad] &= np.uint16(0xBFFF)
        return b
    b = rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)
    bad = (b & 0x7F800000) == 0x7F800000
    b[bad] &= np.uint32(0xBFFFFFFF)
    return b.view(np.float32)


def hub_positions(wl: Workload, seed: int = 0) -> np.ndarray:
    if wl.n_hubs <= 0 or wl.hub_mode is None:
        return np.zeros(0, dtype=np.int64)
    rng = layer_seed(wl, seed, 0, 3)
    hi = max(1, wl.n_prefix)
    cand = np.arange(1, hi, dtype=np.int64)
    n = min(wl.n_hubs, cand.size)
    return np.sort(rng.choice(cand, size=n, replace=False))


def hub_layer_set(wl: Workload, seed: int = 0) -> np.ndarray:
    if wl.hub_layers is None:
        return np.arange(wl.n_layers)
    rng = layer_seed(wl, seed, 0, 3, 1)
    return np.sort(rng.choice(wl.n_layers, size=min(wl.hub_layers, wl.n_layers), replace=False))


def _queries_f64(wl: Workload, seed: int, layer: int) -> np.ndarray:
    shape = (wl.batch, wl.n_q_heads, wl.window, wl.head_dim)
    if wl.query_model == "zero":
        return np.zeros(shape)
    q = layer_seed(wl, seed, layer, 0).standard_normal(shape)
    if wl.rope_base is not None:
        pos = np.arange(wl.n_keys - wl.window, wl.n_keys)
        q = _rope(q, pos, wl.rope_base)
    return q


def _group_directions(wl: Workload, q64: np.ndarray) -> np.ndarray:
    """u[b, g]: unit mean of KV group g's window queries (post-RoPE, fp64)."""
    B, Hq, w, d = q64.shape
    G = wl.group
    m = q64.reshape(B, wl.n_kv_heads, G * w, d).mean(axis=2)
    n = np.linalg.norm(m, axis=-1, keepdims=True)
    e0 = np.zeros(d)
    e0[0] = 1.0
    return np.where(n > 0, m / np.where(n > 0, n, 1.0), e0)


def _key_block(wl: Workload, seed: int, layer: int, b: int, g: int, blk: int,
               u: np.ndarray, hubs: np.ndarray, hubs_on: bool, ar_state):
    j0 = blk * KEY_BLOCK
    j1 = min(wl.n_keys, j0 + KEY_BLOCK)
    n, d = j1 - j0, wl.head_dim
    rng = layer_seed(wl, seed, layer, 1, b, g, blk)
    if wl.key_model == "const":
        base = layer_seed(wl, seed, layer, 1, b, g).standard_normal(d)
        k = np.broadcast_to(base, (n, d)).copy()
    elif wl.key_model == "ar1":
        rho = wl.ar_rho
        x = rng.standard_normal((n, d)) * math.sqrt(1.0 - rho * rho)
        if ar_state is None:  # stationary start: k_0 ~ N(0, 1)
            x[0] /= math.sqrt(1.0 - rho * rho)
            k = _ar_scan(x, rho, np.zeros(d))
        else:
            k = _ar_scan(x, rho, ar_state)
        ar_state = k[-1].copy()
    else:
        k = rng.standard_normal((n, d))
    if wl.k_mult != 1.0:
        k *= wl.k_mult
    if wl.layer_k_mult is not None:
        k *= wl.layer_k_mult[layer]
    if wl.rope_base is not None:
        k = _rope(k, np.arange(j0, j1), wl.rope_base)
    if hubs_on and hubs.size:
        sel = hubs[(hubs >= j0) & (hubs < j1)] - j0
        if sel.size:
            if wl.hub_mode == "mean_query":
                nrm = np.linalg.norm(k[sel], axis=-1, keepdims=True)
                k[sel] = wl.hub_scale * nrm * u[None, :]
            else:
                k[sel] *= wl.hub_scale
    if wl.sink and j0 == 0:
        k[0] = wl.sink_scale * math.sqrt(d) * u
    return k, ar_state


def _ar_scan(x: np.ndarray, rho: float, prev: np.ndarray) -> np.ndarray:
    """y_t = rho * y_{t-1} + x_t with y_{-1} = prev (sequential, fp64)."""
    from scipy.signal import lfilter

    zi = (rho * prev)[None, :]
    y, _ = lfilter([1.0], [1.0, -rho], x, axis=0, zi=zi)
    return y


def _threads(threads: Optional[int]) -> int:
    if threads is not None:
        return max(1, threads)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(wl: Workload, seed: int = 0, layers: Optional[Iterable[int]] = None,
                with_v: bool = True, with_hidden: bool = True,
                threads: Optional[int] = None) -> dict:
    """Build the host arrays of one workload.

    Returns a dict with ``q`` [L, B, Hq, w, d], ``k`` and ``v`` [L, B, Hkv, N, d]
    (uint16 bf16 bits, or float32), ``hidden`` [B, N, hidden_dim] (uint16) for
    workloads with a token-set budget, and the hub metadata. ``layers`` picks a
    subset of layers (in the given order); their content does not depend on
    which other layers are generated.
    """
    layers = list(range(wl.n_layers)) if layers is None else list(layers)
    L, B, Hq, Hkv, N, w, d = len(layers), wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_keys, wl.window, wl.head_dim
    et = np.uint16 if wl.dtype == "bf16" else np.float32
    q = np.empty((L, B, Hq, w, d), dtype=et)
    k = np.empty((L, B, Hkv, N, d), dtype=et)
    v = np.empty((L, B, Hkv, N, d), dtype=et) if with_v else None
    hubs = hub_positions(wl, seed)
    hub_layers = set(int(x) for x in hub_layer_set(wl, seed))
    nblk = (N + KEY_BLOCK - 1) // KEY_BLOCK

    dirs = {}
    for li, layer in enumerate(layers):
        q64 = _queries_f64(wl, seed, layer)
        q[li] = _round(wl, q64)
        dirs[li] = _group_directions(wl, q64)

    def key_slab(li, layer, b, g):
        state = None
        for blk in range(nblk):
            kb, state = _key_block(wl, seed, layer, b, g, blk, dirs[li][b, g], hubs,
                                   layer in hub_layers, state)
            j0 = blk * KEY_BLOCK
            k[li, b, g, j0:j0 + kb.shape[0]] = _round(wl, kb)

    def value_slab(li, layer, b, g):
        rng = layer_seed(wl, seed, layer, 2, b, g)
        v[li, b, g] = _random_finite_bits(rng, (N, d), wl.dtype)

    jobs = [(li, layer, b, g) for li, layer in enumerate(layers) for b in range(B) for g in range(Hkv)]
    nthr = _threads(threads)
    # fp64 temporaries are a few times one key block per worker
    with cf.ThreadPoolExecutor(nthr) as ex:
        list(ex.map(lambda a: key_slab(*a), jobs))
        if with_v:
            list(ex.map(lambda a: value_slab(*a), jobs))

    hidden = None
    if with_hidden and wl.hidden_dim:
        hidden = np.empty((B, N, wl.hidden_dim), dtype=np.uint16)
        for b in range(B):
            hidden[b] = _random_finite_bits(layer_seed(wl, seed, 0, 4, b), (N, wl.hidden_dim), "bf16")

    return {
        "q": q, "k": k, "v": v, "hidden": hidden,
        "layers": layers, "hub_pos": hubs, "hub_layers": sorted(hub_layers),
        "seed": seed,
    }
