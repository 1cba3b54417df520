"""ctypes binding of libkvsel (argument marshalling only).

Every function here forwards torch tensors' device pointers, sizes and strides
to the C ABI declared in ``include/kvsel.h`` and raises ``KvselError`` on a
non-zero status. All arithmetic runs in the library's HIP kernels; PyTorch
only provides device memory and the current HIP stream. If the library is not
built the first call raises ``RuntimeError``: there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvsel.so")

KVSEL_OK = 0
KVSEL_ERR_INVALID_ARG = 1
KVSEL_ERR_UNSUPPORTED = 2
KVSEL_ERR_WORKSPACE = 3
KVSEL_ERR_HIP = 4
KVSEL_ERR_TOO_LARGE = 5
KVSEL_TOPK_NOALLOC_MAX_BYTES = 16 << 20

KVSEL_DTYPE_F32 = 0
KVSEL_DTYPE_BF16 = 1
KVSEL_POOL_AVG = 0
KVSEL_POOL_MAX = 1
KVSEL_ACC_ADD = 0
KVSEL_ACC_HEAD_MEAN = 1
KVSEL_PATH_AUTO = 0
KVSEL_PATH_STREAM = 1
KVSEL_PATH_GENERAL = 2

EXPORTED = (
    "kvsel_score_workspace_bytes",
    "kvsel_score_path",
    "kvsel_score",
    "kvsel_score_lse",
    "kvsel_score_stats",
    "kvsel_layer_summary",
    "kvsel_pivot_layer",
    "kvsel_accumulate",
    "kvsel_topk_workspace_bytes",
    "kvsel_topk",
    "kvsel_topk_sinks",
    "kvsel_topk_noalloc",
    "kvsel_gather",
    "kvsel_csm_candidates",
    "kvsel_csm_workspace_bytes",
    "kvsel_csm",
    "kvsel_decode_workspace_bytes",
    "kvsel_decode_attention",
    "kvsel_status_string",
    "kvsel_version",
)


class KvselError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class ScoreDesc(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("n_keys", ctypes.c_int64),
        ("pool_kernel", ctypes.c_int32),
        ("pool_type", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_strides", ctypes.c_int64 * 4),
        ("k_strides", ctypes.c_int64 * 4),
        ("path", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libkvsel.so (built in-tree by ``python -m token_selection_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libkvsel.so is not built ({_LIB_PATH}); run python -m token_selection_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kvsel_score_workspace_bytes.argtypes = [ctypes.POINTER(ScoreDesc)]
    lib.kvsel_score_workspace_bytes.restype = sz
    lib.kvsel_score_path.argtypes = [ctypes.POINTER(ScoreDesc)]
    lib.kvsel_score_path.restype = i32
    lib.kvsel_score.argtypes = [ctypes.POINTER(ScoreDesc), vp, vp, vp, i32, vp, vp, sz, vp]
    lib.kvsel_score.restype = i32
    lib.kvsel_score_lse.argtypes = [ctypes.POINTER(ScoreDesc), vp, vp, vp, vp, i32, vp, sz, vp]
    lib.kvsel_score_stats.argtypes = [ctypes.POINTER(ScoreDesc), vp, vp, vp, i32, vp, ctypes.c_float, vp, vp, vp, vp,
                                      sz, vp]
    lib.kvsel_score_stats.restype = i32
    lib.kvsel_layer_summary.argtypes = [i32, i32, i32, i64, vp, vp, vp, vp, vp]
    lib.kvsel_layer_summary.restype = i32
    lib.kvsel_pivot_layer.argtypes = [i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                      ctypes.c_float, ctypes.c_float, ctypes.POINTER(i32)]
    lib.kvsel_pivot_layer.restype = i32
    lib.kvsel_score_lse.restype = i32
    lib.kvsel_accumulate.argtypes = [i32, i32, i64, vp, vp, i32, vp]
    lib.kvsel_accumulate.restype = i32
    lib.kvsel_topk_workspace_bytes.argtypes = [i32, i32, i64, i32, i32]
    lib.kvsel_topk_workspace_bytes.restype = sz
    lib.kvsel_topk.argtypes = [i32, i32, i64, i32, i32, vp, vp, vp, sz, vp]
    lib.kvsel_topk.restype = i32
    lib.kvsel_topk_sinks.argtypes = [i32, i32, i64, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.kvsel_topk_sinks.restype = i32
    lib.kvsel_topk_noalloc.argtypes = [i32, i32, i64, i32, i32, i32, vp, vp, vp]
    lib.kvsel_topk_noalloc.restype = i32
    lib.kvsel_gather.argtypes = [i32, i32, i32, i32, i32, i64, i64, vp, ctypes.POINTER(ctypes.c_int64), vp, vp, vp]
    lib.kvsel_gather.restype = i32
    lib.kvsel_csm_candidates.argtypes = [i64, i32, i32, i32]
    lib.kvsel_csm_candidates.restype = i64
    lib.kvsel_csm_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.kvsel_csm_workspace_bytes.restype = sz
    lib.kvsel_csm.argtypes = [i32, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kvsel_csm.restype = i32
    lib.kvsel_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i64]
    lib.kvsel_decode_workspace_bytes.restype = sz
    lib.kvsel_decode_attention.argtypes = [i32, i32, i32, i32, i64, ctypes.c_float, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kvsel_decode_attention.restype = i32
    lib.kvsel_status_string.argtypes = [i32]
    lib.kvsel_status_string.restype = ctypes.c_char_p
    lib.kvsel_version.argtypes = []
    lib.kvsel_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kvsel_status_string(int(status)).decode()


def version() -> str:
    return load_library().kvsel_version().decode()


def _check(status: int, where: str) -> None:
    if status != KVSEL_OK:
        raise KvselError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KVSEL_DTYPE_BF16
    if dt == torch.float32:
        return KVSEL_DTYPE_F32
    raise KvselError(KVSEL_ERR_UNSUPPORTED, f"dtype {dt}")


def budget_from_rate(rate: float, n_keys: int, window: int) -> int:
    """Kept count for a retention rate: ceil(rate * N) clamped to [window, N]."""
    b = int(math.ceil(rate * n_keys - 1e-9))
    return max(window, min(n_keys, b))


# ---------------------------------------------------------------------------
# score
# ---------------------------------------------------------------------------
def _as5(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dim() == 4:
        return t.unsqueeze(0)
    if t.dim() != 5:
        raise ValueError(f"{name} must be [L, B, H, T, d] or [B, H, T, d]")
    return t


def score_desc(q_win: torch.Tensor, k: torch.Tensor, window: int, pool_kernel: int = 7,
               softmax_scale: float = 0.0, pool_type: int = 0, path: int = KVSEL_PATH_AUTO) -> ScoreDesc:
    q5, k5 = _as5(q_win, "q_win"), _as5(k, "k")
    L, B, Hq, w, d = q5.shape
    Lk, Bk, Hkv, N, dk = k5.shape
    if (Lk, Bk, dk) != (L, B, d) or w != window:
        raise ValueError("q_win [L,B,Hq,w,d] and k [L,B,Hkv,N,d] disagree")
    if q5.stride(-1) != 1 or k5.stride(-1) != 1:
        raise ValueError("head dimension must be contiguous")
    desc = ScoreDesc()
    desc.n_layers, desc.batch, desc.n_q_heads, desc.n_kv_heads = L, B, Hq, Hkv
    desc.head_dim, desc.window, desc.n_keys = d, window, N
    desc.pool_kernel, desc.pool_type = pool_kernel, int(pool_type)
    desc.dtype = _dtype_code(q5.dtype)
    if k5.dtype != q5.dtype:
        raise ValueError("q_win and k must share a dtype")
    desc.softmax_scale = float(softmax_scale)
    for i in range(4):
        desc.q_strides[i] = q5.stride(i)
        desc.k_strides[i] = k5.stride(i)
    desc.path = int(path)
    desc.reserved = 0
    return desc


def kvsel_score_workspace_bytes(desc: ScoreDesc) -> int:
    return int(load_library().kvsel_score_workspace_bytes(ctypes.byref(desc)))


def kvsel_score_path(desc: ScoreDesc) -> int:
    """KVSEL_PATH_STREAM or KVSEL_PATH_GENERAL: the kernels a scoring call with
    ``desc`` runs (-1: invalid, or the streaming kernels asked for a shape
    they do not take)."""
    return int(load_library().kvsel_score_path(ctypes.byref(desc)))


def kvsel_score(q_win: torch.Tensor, k: torch.Tensor, scores: Optional[torch.Tensor] = None, *, window: int,
                pool_kernel: int = 7, accumulate: bool = False, lse_out: Optional[torch.Tensor] = None,
                softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None, stream=None,
                desc: Optional[ScoreDesc] = None, pool_type: int = 0, path: int = KVSEL_PATH_AUTO) -> torch.Tensor:
    """Saliency scores [B, Hkv, N - w] (fp32), summed over the L layers of the
    call (added to ``scores`` when ``accumulate``). ``q_win``: [L, B, Hq, w, d]
    or [B, Hq, w, d]; ``k``: [L, B, Hkv, N, d] or [B, Hkv, N, d]; bf16 or fp32.
    ``path`` picks the scoring kernels (KVSEL_PATH_*), used when ``desc`` is
    not given."""
    lib = load_library()
    if desc is None:
        desc = score_desc(q_win, k, window, pool_kernel, softmax_scale, pool_type, path)
    B, Hkv, N, w = desc.batch, desc.n_kv_heads, desc.n_keys, desc.window
    dev = k.device
    if scores is None:
        scores = torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev)
    if scores.dtype != torch.float32 or not scores.is_contiguous() or tuple(scores.shape) != (B, Hkv, N - w):
        raise ValueError("scores must be a contiguous float32 [B, Hkv, N - w] tensor")
    if lse_out is not None and (lse_out.dtype != torch.float32 or not lse_out.is_contiguous() or
                                lse_out.numel() != desc.n_layers * B * desc.n_q_heads * w):
        raise ValueError("lse_out must be a contiguous float32 [L, B, Hq, w] tensor")
    need = int(lib.kvsel_score_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.kvsel_score(ctypes.byref(desc), _ptr(q_win), _ptr(k), _ptr(scores), 1 if accumulate else 0,
                         _ptr(lse_out), _ptr(workspace), workspace.numel(), _stream(dev, stream))
    _check(st, "kvsel_score")
    return scores


def kvsel_score_lse(q_win: torch.Tensor, k: torch.Tensor, lse_in: torch.Tensor,
                    scores: Optional[torch.Tensor] = None, *, window: int, pool_kernel: int = 7,
                    accumulate: bool = False, softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                    stream=None, desc: Optional[ScoreDesc] = None, pool_type: int = 0,
                    path: int = KVSEL_PATH_AUTO) -> torch.Tensor:
    """As kvsel_score, with the natural-log LSE of every window row handed in
    (``lse_in``: contiguous float32 [L, B, Hq, w]); only the second softmax
    pass runs."""
    lib = load_library()
    if desc is None:
        desc = score_desc(q_win, k, window, pool_kernel, softmax_scale, pool_type, path)
    B, Hkv, N, w = desc.batch, desc.n_kv_heads, desc.n_keys, desc.window
    dev = k.device
    if scores is None:
        scores = torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev)
    if scores.dtype != torch.float32 or not scores.is_contiguous() or tuple(scores.shape) != (B, Hkv, N - w):
        raise ValueError("scores must be a contiguous float32 [B, Hkv, N - w] tensor")
    if (lse_in.dtype != torch.float32 or not lse_in.is_contiguous() or
            lse_in.numel() != desc.n_layers * B * desc.n_q_heads * w):
        raise ValueError("lse_in must be a contiguous float32 [L, B, Hq, w] tensor")
    need = int(lib.kvsel_score_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.kvsel_score_lse(ctypes.byref(desc), _ptr(q_win), _ptr(k), _ptr(lse_in), _ptr(scores),
                             1 if accumulate else 0, _ptr(workspace), workspace.numel(), _stream(dev, stream))
    _check(st, "kvsel_score_lse")
    return scores


def kvsel_score_stats(q_win: torch.Tensor, k: torch.Tensor, scores: Optional[torch.Tensor] = None, *, window: int,
                      small_p: float, pool_kernel: int = 7, accumulate: bool = False, lse_out=None,
                      softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None, stream=None,
                      desc: Optional[ScoreDesc] = None, pool_type: int = 0, path: int = KVSEL_PATH_AUTO,
                      out=None):
    """As kvsel_score, also returning every window row's attention entropy,
    sum of p^2 and count of keys with p < small_p ([L, B, Hq, w] each):
    (scores, entropy, sum_p2, n_below). ``out`` = (entropy, sum_p2, n_below)
    preallocated (float32, float32, int32 [L, B, Hq, w], contiguous)."""
    lib = load_library()
    if desc is None:
        desc = score_desc(q_win, k, window, pool_kernel, softmax_scale, pool_type, path)
    L, B, Hq, Hkv, N, w = desc.n_layers, desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.n_keys, desc.window
    dev = k.device
    if scores is None:
        scores = torch.empty((B, Hkv, N - w), dtype=torch.float32, device=dev)
    if scores.dtype != torch.float32 or not scores.is_contiguous() or tuple(scores.shape) != (B, Hkv, N - w):
        raise ValueError("scores must be a contiguous float32 [B, Hkv, N - w] tensor")
    if lse_out is not None and (lse_out.dtype != torch.float32 or not lse_out.is_contiguous() or
                                lse_out.numel() != L * B * Hq * w):
        raise ValueError("lse_out must be a contiguous float32 [L, B, Hq, w] tensor")
    if out is None:
        entropy = torch.empty((L, B, Hq, w), dtype=torch.float32, device=dev)
        sum_p2 = torch.empty_like(entropy)
        n_below = torch.empty((L, B, Hq, w), dtype=torch.int32, device=dev)
    else:
        entropy, sum_p2, n_below = out
        for t, dt in ((entropy, torch.float32), (sum_p2, torch.float32), (n_below, torch.int32)):
            if tuple(t.shape) != (L, B, Hq, w) or t.dtype != dt or not t.is_contiguous():
                raise ValueError("out must be contiguous [L, B, Hq, w] tensors (float32, float32, int32)")
    need = int(lib.kvsel_score_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.kvsel_score_stats(ctypes.byref(desc), _ptr(q_win), _ptr(k), _ptr(scores), 1 if accumulate else 0,
                               _ptr(lse_out), float(small_p), _ptr(entropy), _ptr(sum_p2), _ptr(n_below),
                               _ptr(workspace), workspace.numel(), _stream(dev, stream))
    _check(st, "kvsel_score_stats")
    return scores, entropy, sum_p2, n_below


def kvsel_layer_summary(entropy: torch.Tensor, sum_p2: torch.Tensor, n_below: torch.Tensor, *, n_keys: int,
                        stream=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-layer means [L, 3] (entropy, sparsity, variance) of kvsel_score_stats'
    row statistics [L, B, Hq, w]."""
    lib = load_library()
    for t, dt in ((entropy, torch.float32), (sum_p2, torch.float32), (n_below, torch.int32)):
        if t.dim() != 4 or t.dtype != dt or not t.is_contiguous() or t.shape != entropy.shape:
            raise ValueError("statistics must be contiguous [L, B, Hq, w] tensors (float32, float32, int32)")
    L, B, Hq, w = entropy.shape
    if out is None:
        out = torch.empty((L, 3), dtype=torch.float32, device=entropy.device)
    if tuple(out.shape) != (L, 3) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [L, 3] tensor")
    _check(lib.kvsel_layer_summary(L, B * Hq * w, w, n_keys, _ptr(entropy), _ptr(sum_p2), _ptr(n_below), _ptr(out),
                                   _stream(entropy.device, stream)), "kvsel_layer_summary")
    return out


def kvsel_pivot_layer(mean_entropy, mean_sparsity, *, min_drop: float, min_rise: float) -> int:
    """StructKV's pivot layer from per-layer means (host sequences of floats)."""
    lib = load_library()
    e = [float(x) for x in mean_entropy]
    sp = [float(x) for x in mean_sparsity]
    if len(e) != len(sp):
        raise ValueError("one entropy and one sparsity value per layer")
    ea = (ctypes.c_float * max(len(e), 1))(*e)
    sa = (ctypes.c_float * max(len(sp), 1))(*sp)
    out = ctypes.c_int32(-1)
    _check(lib.kvsel_pivot_layer(len(e), ea, sa, min_drop, min_rise, ctypes.byref(out)), "kvsel_pivot_layer")
    return int(out.value)


# ---------------------------------------------------------------------------
# CentroidKV chunked soft matching, decode attention
# ---------------------------------------------------------------------------
def csm_merge_count(rate: float, n_tokens: int, n_sink: int, n_recent: int) -> int:
    """Merges of one round at compression ratio ``rate`` (a fraction of the
    middle tokens; the progressive schedule lowers it linearly per round)."""
    return int(math.floor(rate * (n_tokens - n_sink - n_recent) + 1e-9))


def kvsel_csm(k: torch.Tensor, v: torch.Tensor, degree: Optional[torch.Tensor] = None, *, chunk: int,
              n_sink: int, n_recent: int, n_merge: int, with_decisions: bool = False, stream=None):
    """One CSM round over the slabs of k, v ([..., n, d] bf16, contiguous):
    returns (k_out, v_out, degree_out) with n - n_merge rows per slab, plus
    (score, match, chosen) with ``with_decisions``."""
    lib = load_library()
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or not k.is_contiguous() or not v.is_contiguous():
        raise ValueError("k and v must be contiguous bf16 tensors")
    if k.shape != v.shape or k.dim() < 2:
        raise ValueError("k and v must have the same [..., n, d] shape")
    n, d = k.shape[-2], k.shape[-1]
    lead = tuple(k.shape[:-2])
    S = int(math.prod(lead)) if lead else 1
    if degree is not None and (degree.dtype != torch.int32 or not degree.is_contiguous() or
                               tuple(degree.shape) != lead + (n,)):
        raise ValueError("degree must be a contiguous int32 [..., n] tensor")
    cand = int(lib.kvsel_csm_candidates(n, chunk, n_sink, n_recent))
    if cand < 0:
        raise ValueError("invalid CSM sizes (chunk even in 2..64, 0 <= n_sink, n_recent, n_sink + n_recent <= n)")
    if not (0 <= n_merge <= cand):
        raise ValueError(f"n_merge must be in [0, {cand}] (A tokens with a partner)")
    n_out = n - n_merge
    dev = k.device
    k_out = torch.empty(lead + (n_out, d), dtype=k.dtype, device=dev)
    v_out = torch.empty_like(k_out)
    deg_out = torch.empty(lead + (n_out,), dtype=torch.int32, device=dev)
    n_a = cand + (1 if cand >= 0 and (n - n_sink - n_recent) % chunk == 1 else 0)
    score = match = chosen = None
    if with_decisions:
        score = torch.empty(lead + (max(n_a, 0),), dtype=torch.float32, device=dev)
        match = torch.empty(lead + (max(n_a, 0),), dtype=torch.int32, device=dev)
        chosen = torch.empty(lead + (max(n_merge, 0),), dtype=torch.int32, device=dev)
    need = int(lib.kvsel_csm_workspace_bytes(S, n, chunk, n_sink, n_recent, n_merge))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.kvsel_csm(S, n, d, chunk, n_sink, n_recent, n_merge, _ptr(k), _ptr(v), _ptr(degree), _ptr(k_out),
                         _ptr(v_out), _ptr(deg_out), _ptr(score), _ptr(match), _ptr(chosen), _ptr(ws), ws.numel(),
                         _stream(dev, stream)), "kvsel_csm")
    if with_decisions:
        return k_out, v_out, deg_out, score, match, chosen
    return k_out, v_out, deg_out


def kvsel_decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, n_keys: int) -> int:
    return int(load_library().kvsel_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, n_keys))


def kvsel_decode_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, degree: Optional[torch.Tensor] = None,
                           *, softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step: q [B, Hq, d] bf16 against k, v [B, Hkv, n, d] bf16
    (and degree [B, Hkv, n] int32) -> out [B, Hq, d] float32."""
    lib = load_library()
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("q, k and v must be contiguous bf16 tensors")
    B, Hq, d = q.shape
    _, Hkv, n, _ = k.shape
    if tuple(k.shape) != (B, Hkv, n, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, n, d]")
    if degree is not None and (degree.dtype != torch.int32 or not degree.is_contiguous() or
                               tuple(degree.shape) != (B, Hkv, n)):
        raise ValueError("degree must be a contiguous int32 [B, Hkv, n] tensor")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    need = int(lib.kvsel_decode_workspace_bytes(B, Hq, Hkv, d, n))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.kvsel_decode_attention(B, Hq, Hkv, d, n, softmax_scale, _ptr(q), _ptr(k), _ptr(v), _ptr(degree),
                                      _ptr(out), _ptr(workspace), workspace.numel(), _stream(q.device, stream)),
           "kvsel_decode_attention")
    return out


# ---------------------------------------------------------------------------
# accumulate
# ---------------------------------------------------------------------------
def kvsel_accumulate(src: torch.Tensor, dst: Optional[torch.Tensor] = None, mode: int = KVSEL_ACC_ADD,
                     stream=None) -> torch.Tensor:
    """ADD: dst [B, H, n] += src. HEAD_MEAN: dst [B, 1, n] = mean over heads of src [B, H, n]."""
    lib = load_library()
    if src.dim() != 3 or src.dtype != torch.float32 or not src.is_contiguous():
        raise ValueError("src must be a contiguous float32 [B, H, n] tensor")
    B, H, n = src.shape
    shape = (B, H, n) if mode == KVSEL_ACC_ADD else (B, 1, n)
    if dst is None:
        if mode == KVSEL_ACC_ADD:
            raise ValueError("ADD needs a destination")
        dst = torch.empty(shape, dtype=torch.float32, device=src.device)
    if tuple(dst.shape) != shape or dst.dtype != torch.float32 or not dst.is_contiguous():
        raise ValueError(f"dst must be a contiguous float32 {shape} tensor")
    _check(lib.kvsel_accumulate(B, H, n, _ptr(src), _ptr(dst), mode, _stream(src.device, stream)),
           "kvsel_accumulate")
    return dst


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------
def kvsel_topk_workspace_bytes(batch: int, rows: int, n_keys: int, window: int, budget: int) -> int:
    return int(load_library().kvsel_topk_workspace_bytes(batch, rows, n_keys, window, budget))


def kvsel_topk(scores: torch.Tensor, *, n_keys: int, window: int, budget: int, idx: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None, n_sink: int = 0) -> torch.Tensor:
    """Kept positions [B, rows, budget] (int32, ascending, window last) of
    scores [B, rows, N - w]; with ``n_sink`` > 0 positions 0 .. n_sink-1 are
    always kept (kvsel_topk_sinks)."""
    lib = load_library()
    if scores.dim() != 3 or scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 [B, rows, N - w] tensor")
    B, rows, n_prefix = scores.shape
    if n_prefix != n_keys - window:
        raise ValueError("scores length must be n_keys - window")
    if idx is None:
        idx = torch.empty((B, rows, budget), dtype=torch.int32, device=scores.device)
    if tuple(idx.shape) != (B, rows, budget) or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 [B, rows, budget] tensor")
    need = int(lib.kvsel_topk_workspace_bytes(B, rows, n_keys, window, budget))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    if n_sink:
        _check(lib.kvsel_topk_sinks(B, rows, n_keys, window, budget, n_sink, _ptr(scores), _ptr(idx),
                                    _ptr(workspace), ws_bytes, _stream(scores.device, stream)), "kvsel_topk_sinks")
    else:
        _check(lib.kvsel_topk(B, rows, n_keys, window, budget, _ptr(scores), _ptr(idx), _ptr(workspace), ws_bytes,
                              _stream(scores.device, stream)), "kvsel_topk")
    return idx


def kvsel_topk_noalloc(scores: torch.Tensor, idx: torch.Tensor, *, n_keys: int, window: int, budget: int,
                       n_sink: int = 0, stream=None) -> torch.Tensor:
    """kvsel_topk without a workspace: the library's static per-GPU scratch
    serves (calls that overlap on one GPU race). ``idx`` [B, rows, budget]
    int32 must be given, so the call allocates nothing."""
    lib = load_library()
    if scores.dim() != 3 or scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 [B, rows, N - w] tensor")
    B, rows, n_prefix = scores.shape
    if n_prefix != n_keys - window:
        raise ValueError("scores length must be n_keys - window")
    if tuple(idx.shape) != (B, rows, budget) or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 [B, rows, budget] tensor")
    _check(lib.kvsel_topk_noalloc(B, rows, n_keys, window, budget, n_sink, _ptr(scores), _ptr(idx),
                                  _stream(scores.device, stream)), "kvsel_topk_noalloc")
    return idx


# ---------------------------------------------------------------------------
# gather
# ---------------------------------------------------------------------------
def kvsel_gather(src: torch.Tensor, idx: torch.Tensor, dst: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """Bit-exact row gather. ``src``: [L, B, H, N, *row] or [B, H, N, *row]
    (row dims contiguous); ``idx``: [B, 1 or H, budget] int32. Returns
    [L, B, H, budget, *row] (or without L)."""
    lib = load_library()
    if idx.dim() != 3 or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 [B, 1 or H, budget] tensor")
    B, idx_heads, budget = idx.shape
    # split src into (L, B, H, N) + row
    if src.dim() < 4:
        raise ValueError("src must have at least [B, H, N, row] dims")
    five = src.dim() >= 5
    lead = 4 if five else 3
    row_shape = tuple(src.shape[lead:])
    row_elems = 1
    for s_ in row_shape:
        row_elems *= s_
    # row dims must be contiguous
    expect = 1
    for dim in range(src.dim() - 1, lead - 1, -1):
        if src.shape[dim] != 1 and src.stride(dim) != expect:
            raise ValueError("row dims of src must be contiguous")
        expect *= src.shape[dim]
    es = src.element_size()
    if five:
        L, Bs, H, N = src.shape[:4]
        strides = [src.stride(i) * es for i in range(4)]
    else:
        L = 1
        Bs, H, N = src.shape[:3]
        strides = [0] + [src.stride(i) * es for i in range(3)]
    if Bs != B:
        raise ValueError("src and idx batch differ")
    out_shape = ((L,) if five else ()) + (B, H, budget) + row_shape
    if dst is None:
        dst = torch.empty(out_shape, dtype=src.dtype, device=src.device)
    if tuple(dst.shape) != out_shape or dst.dtype != src.dtype or not dst.is_contiguous():
        raise ValueError(f"dst must be a contiguous {out_shape} tensor of src's dtype")
    arr = (ctypes.c_int64 * 4)(*strides)
    _check(lib.kvsel_gather(L, B, H, idx_heads, budget, N, row_elems * es, _ptr(src), arr, _ptr(idx), _ptr(dst),
                            _stream(src.device, stream)), "kvsel_gather")
    return dst
