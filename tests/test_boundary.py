"""The C-ABI library: it loads, exports every function include/kvsel.h
declares, its struct layout matches the binding, and every argument error is
reported before any launch (these calls never reach the GPU). The host-only
pivot rule is checked against the oracle here. CPU only."""

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")

kvsel = pytest.importorskip("token_selection_amd.kvsel")


@pytest.fixture(scope="module")
def lib():
    return kvsel.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(kvsel.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", kvsel.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kvsel_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_struct_layout_matches_header():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "kvsel.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(kvsel_score_desc_t), offsetof(kvsel_score_desc_t, n_keys),
         offsetof(kvsel_score_desc_t, pool_kernel), offsetof(kvsel_score_desc_t, softmax_scale),
         offsetof(kvsel_score_desc_t, q_strides), offsetof(kvsel_score_desc_t, k_strides),
         offsetof(kvsel_score_desc_t, path), offsetof(kvsel_score_desc_t, reserved));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    D = kvsel.ScoreDesc
    assert got == [ctypes.sizeof(D), D.n_keys.offset, D.pool_kernel.offset, D.softmax_scale.offset,
                   D.q_strides.offset, D.k_strides.offset, D.path.offset, D.reserved.offset]


def test_status_strings(lib):
    for code in range(6):
        assert kvsel.status_string(code).startswith("KVSEL")
    assert "unknown" in kvsel.status_string(99)
    assert "gfx950" in kvsel.version()


def good_desc(**kw):
    d = kvsel.ScoreDesc()
    d.n_layers, d.batch, d.n_q_heads, d.n_kv_heads = 1, 1, 8, 2
    d.head_dim, d.window, d.n_keys = 128, 8, 1024
    d.pool_kernel, d.pool_type, d.dtype, d.softmax_scale = 7, 0, kvsel.KVSEL_DTYPE_BF16, 0.0
    q = [4 * 8 * 128, 4 * 8 * 128, 8 * 128, 128]
    k = [2 * 1024 * 128, 2 * 1024 * 128, 1024 * 128, 128]
    for i in range(4):
        d.q_strides[i] = q[i]
        d.k_strides[i] = k[i]
    for key, v in kw.items():
        if key in ("q_strides", "k_strides"):
            for i in range(4):
                getattr(d, key)[i] = v[i]
        else:
            setattr(d, key, v)
    return d


FAKE = 1 << 32  # a 256-byte aligned address that is never dereferenced


@pytest.mark.parametrize("field,value,status", [
    ("n_layers", 0, 1), ("batch", 0, 1), ("n_q_heads", 7, 1), ("n_kv_heads", 0, 1),
    ("window", 0, 1), ("n_keys", 4, 1), ("n_keys", 1 << 31, 1),
    ("pool_kernel", 4, 1), ("pool_kernel", 0, 1), ("pool_kernel", 257, 1),
    ("softmax_scale", float("inf"), 1), ("softmax_scale", float("nan"), 1),
    ("head_dim", 96, 2), ("dtype", 7, 2), ("pool_type", 2, 2),
    ("k_strides", [0, 0, 1024 * 128, 127], 1), ("q_strides", [0, 0, -128, 128], 1),
    ("path", 3, 1), ("path", -1, 1), ("reserved", 1, 1),
])
def test_score_rejects_bad_descriptor(lib, field, value, status):
    d = good_desc(**{field: value})
    assert lib.kvsel_score_workspace_bytes(ctypes.byref(d)) == 0
    st = lib.kvsel_score(ctypes.byref(d), FAKE, FAKE, FAKE, 0, None, FAKE, 1 << 40, None)
    assert st == status


def test_score_path_field(lib):
    """The explicit path field: AUTO resolves to the streaming kernels for a
    bf16 head_dim-128 shape and to the general ones for fp32, head_dim 64
    with w > 256 is general only, and an explicit streaming choice on a shape
    it does not take resolves to -1 and is refused with UNSUPPORTED before
    any launch."""
    S, G, A = kvsel.KVSEL_PATH_STREAM, kvsel.KVSEL_PATH_GENERAL, kvsel.KVSEL_PATH_AUTO
    assert lib.kvsel_score_path(ctypes.byref(good_desc())) == S
    assert lib.kvsel_score_path(ctypes.byref(good_desc(path=S))) == S
    assert lib.kvsel_score_path(ctypes.byref(good_desc(path=G))) == G
    f32 = dict(dtype=kvsel.KVSEL_DTYPE_F32)
    assert lib.kvsel_score_path(ctypes.byref(good_desc(**f32))) == G
    assert lib.kvsel_score_path(ctypes.byref(good_desc(path=G, **f32))) == G
    assert lib.kvsel_score_path(ctypes.byref(good_desc(path=S, **f32))) == -1
    wide = dict(head_dim=64, window=300, n_keys=1024, q_strides=[4 * 300 * 64, 4 * 300 * 64, 300 * 64, 64],
                k_strides=[2 * 1024 * 64, 2 * 1024 * 64, 1024 * 64, 64])
    assert lib.kvsel_score_path(ctypes.byref(good_desc(path=A, **wide))) == G
    assert lib.kvsel_score_path(ctypes.byref(good_desc(path=S, **wide))) == -1
    assert lib.kvsel_score_path(ctypes.byref(good_desc(path=7))) == -1
    assert lib.kvsel_score_path(None) == -1
    d = good_desc(path=S, **f32)
    need = lib.kvsel_score_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert lib.kvsel_score(ctypes.byref(d), FAKE, FAKE, FAKE, 0, None, FAKE, need, None) == 2


def test_score_rejects_pointers_and_workspace(lib):
    d = good_desc()
    need = lib.kvsel_score_workspace_bytes(ctypes.byref(d))
    assert need > 0 and need % 256 == 0
    assert lib.kvsel_score(None, FAKE, FAKE, FAKE, 0, None, FAKE, need, None) == 1
    assert lib.kvsel_score(ctypes.byref(d), None, FAKE, FAKE, 0, None, FAKE, need, None) == 1
    assert lib.kvsel_score(ctypes.byref(d), FAKE + 8, FAKE, FAKE, 0, None, FAKE, need, None) == 1
    assert lib.kvsel_score(ctypes.byref(d), FAKE, FAKE, None, 0, None, FAKE, need, None) == 1
    assert lib.kvsel_score(ctypes.byref(d), FAKE, FAKE, FAKE, 0, None, None, need, None) == 3
    assert lib.kvsel_score(ctypes.byref(d), FAKE, FAKE, FAKE, 0, None, FAKE, need - 1, None) == 3
    assert lib.kvsel_score(ctypes.byref(d), FAKE, FAKE, FAKE, 0, None, FAKE + 16, need, None) == 3


def test_workspace_grows_with_problem(lib):
    small = lib.kvsel_score_workspace_bytes(ctypes.byref(good_desc()))
    big = lib.kvsel_score_workspace_bytes(ctypes.byref(good_desc(n_layers=4, n_keys=4096,
                                                                 k_strides=[2 * 4096 * 128, 2 * 4096 * 128, 4096 * 128, 128])))
    assert big > small


@pytest.mark.parametrize("args", [
    (0, 1, 100, 4, 10), (1, 0, 100, 4, 10), (1, 1, 100, 0, 10), (1, 1, 100, 4, 3),
    (1, 1, 100, 4, 101), (1, 1, 1 << 31, 4, 10), (1 << 16, 1 << 16, 100, 4, 10),
])
def test_topk_rejects(lib, args):
    B, rows, N, w, budget = args
    assert lib.kvsel_topk(B, rows, N, w, budget, FAKE, FAKE, None, 0, None) == 1


@pytest.mark.parametrize("n_sink", [-1, 7, 1 << 20])
def test_topk_sinks_rejects(lib, n_sink):
    # window 4, budget 10: at most 6 sinks
    need = lib.kvsel_topk_workspace_bytes(1, 1, 100, 4, 10)
    assert lib.kvsel_topk_sinks(1, 1, 100, 4, 10, n_sink, FAKE, FAKE, FAKE, need, None) == 1


def test_max_pool_accepted(lib):
    d = good_desc(pool_type=kvsel.KVSEL_POOL_MAX)
    assert lib.kvsel_score_workspace_bytes(ctypes.byref(d)) > 0


def test_topk_noalloc_rejects(lib):
    """The no-allocation top-k validates like kvsel_topk_sinks, and refuses a
    problem whose scratch exceeds its static array with TOO_LARGE, before any
    launch."""
    assert lib.kvsel_topk_noalloc(1, 2, 1000, 8, 4, 0, FAKE, FAKE, None) == 1        # budget < window
    assert lib.kvsel_topk_noalloc(1, 2, 1000, 8, 100, 93, FAKE, FAKE, None) == 1     # too many sinks
    assert lib.kvsel_topk_noalloc(1, 2, 1000, 8, 100, 0, FAKE, None, None) == 1      # no idx
    assert lib.kvsel_topk_noalloc(0, 2, 1000, 8, 100, 0, FAKE, FAKE, None) == 1
    rows, n = 4000, 1 << 20
    assert lib.kvsel_topk_workspace_bytes(1, rows, n, 8, 100) > kvsel.KVSEL_TOPK_NOALLOC_MAX_BYTES
    assert lib.kvsel_topk_noalloc(1, rows, n, 8, 100, 0, FAKE, FAKE, None) == kvsel.KVSEL_ERR_TOO_LARGE
    assert "no-allocation" in kvsel.status_string(kvsel.KVSEL_ERR_TOO_LARGE)


def test_topk_rejects_null(lib):
    assert lib.kvsel_topk(1, 1, 100, 4, 10, None, FAKE, None, 0, None) == 1
    assert lib.kvsel_topk(1, 1, 100, 4, 10, FAKE, None, None, 0, None) == 1


def test_gather_rejects(lib):
    s = (ctypes.c_int64 * 4)(0, 0, 256, 256)
    ok = (1, 1, 2, 2, 8, 100, 256, FAKE, s, FAKE, FAKE, None)
    bad = [
        (0,) + ok[1:], ok[:1] + (0,) + ok[2:], ok[:3] + (3,) + ok[4:], ok[:4] + (0,) + ok[5:],
        ok[:5] + (0,) + ok[6:], ok[:6] + (0,) + ok[7:], ok[:7] + (None,) + ok[8:],
        ok[:8] + (None,) + ok[9:], ok[:9] + (None,) + ok[10:], ok[:10] + (None,) + ok[11:],
    ]
    for args in bad:
        assert lib.kvsel_gather(*args) == 1
    neg = (ctypes.c_int64 * 4)(0, 0, -256, 256)
    assert lib.kvsel_gather(*(ok[:8] + (neg,) + ok[9:])) == 1


def test_accumulate_rejects(lib):
    assert lib.kvsel_accumulate(1, 1, 10, FAKE, FAKE, 2, None) == 1
    assert lib.kvsel_accumulate(0, 1, 10, FAKE, FAKE, 0, None) == 1
    assert lib.kvsel_accumulate(1, 1, -1, FAKE, FAKE, 0, None) == 1
    assert lib.kvsel_accumulate(1, 1, 10, None, FAKE, 0, None) == 1


def test_rate_helper():
    assert kvsel.budget_from_rate(0.1, 32768, 32) == 3277


def test_topk_workspace_contract(lib):
    need = lib.kvsel_topk_workspace_bytes(1, 8, 131072, 32, 4096)
    assert need > 0 and lib.kvsel_topk_workspace_bytes(1, 8, 131072, 32, 4097 + 131072) == 0
    assert lib.kvsel_topk(1, 8, 131072, 32, 4096, FAKE, FAKE, None, need, None) == 3
    assert lib.kvsel_topk(1, 8, 131072, 32, 4096, FAKE, FAKE, FAKE, need - 1, None) == 3
    assert lib.kvsel_topk(1, 8, 131072, 32, 4096, FAKE, FAKE, FAKE + 16, need, None) == 3


def test_score_lse_rejects(lib):
    d = good_desc()
    need = lib.kvsel_score_workspace_bytes(ctypes.byref(d))
    # missing LSE, then the same descriptor and pointer checks as kvsel_score
    assert lib.kvsel_score_lse(ctypes.byref(d), FAKE, FAKE, None, FAKE, 0, FAKE, need, None) == 1
    assert lib.kvsel_score_lse(None, FAKE, FAKE, FAKE, FAKE, 0, FAKE, need, None) == 1
    assert lib.kvsel_score_lse(ctypes.byref(d), FAKE + 8, FAKE, FAKE, FAKE, 0, FAKE, need, None) == 1
    assert lib.kvsel_score_lse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, FAKE, need - 1, None) == 3
    bad = good_desc(head_dim=96)
    assert lib.kvsel_score_lse(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, None) == 2


def test_score_stats_rejects(lib):
    d = good_desc()
    need = lib.kvsel_score_workspace_bytes(ctypes.byref(d))
    call = lambda desc, p, ent, sp2, nb: lib.kvsel_score_stats(ctypes.byref(desc), FAKE, FAKE, FAKE, 0, None, p,
                                                               ent, sp2, nb, FAKE, need, None)
    for p in (0.0, -1e-3, 1.5, float("nan"), float("inf")):
        assert call(d, p, FAKE, FAKE, FAKE) == 1
    assert call(d, 1e-3, None, FAKE, FAKE) == 1
    assert call(d, 1e-3, FAKE, None, FAKE) == 1
    assert call(d, 1e-3, FAKE, FAKE, None) == 1
    # the statistics ride on the bf16 streaming passes only
    f32 = good_desc(dtype=kvsel.KVSEL_DTYPE_F32, q_strides=[0, 0, 4 * 128, 128], k_strides=[0, 0, 1024 * 128, 128])
    need32 = lib.kvsel_score_workspace_bytes(ctypes.byref(f32))
    assert need32 > 0
    assert lib.kvsel_score_stats(ctypes.byref(f32), FAKE, FAKE, FAKE, 0, None, 1e-3, FAKE, FAKE, FAKE, FAKE, need32,
                                 None) == 2
    assert lib.kvsel_score_stats(ctypes.byref(d), FAKE, FAKE, FAKE, 0, None, 1e-3, FAKE, FAKE, FAKE, FAKE, need - 1,
                                 None) == 3


def test_layer_summary_rejects(lib):
    ok = (2, 64, 16, 1000, FAKE, FAKE, FAKE, FAKE, None)
    assert lib.kvsel_layer_summary(0, *ok[1:]) == 1
    assert lib.kvsel_layer_summary(2, 60, *ok[2:]) == 1      # rows not a multiple of the window
    assert lib.kvsel_layer_summary(2, 64, 16, 15, *ok[4:]) == 1  # fewer keys than the window
    for i in range(4, 8):
        bad = list(ok)
        bad[i] = None
        assert lib.kvsel_layer_summary(*bad) == 1


def _pivot(lib, e, s, drop, rise):
    n = len(e)
    ea = (ctypes.c_float * max(n, 1))(*e)
    sa = (ctypes.c_float * max(n, 1))(*s)
    out = ctypes.c_int32(-7)
    st = lib.kvsel_pivot_layer(n, ea, sa, drop, rise, ctypes.byref(out))
    return st, out.value


def test_pivot_layer_matches_oracle(lib):
    """The host pivot rule against the oracle's, on the same float32 inputs:
    hand-made transitions and seeded random walks."""
    cases = [([10.0, 9.9, 9.8, 6.0, 5.9, 2.0], [0.10, 0.10, 0.12, 0.50, 0.52, 0.90], 0.1, 0.05),
             ([10.0, 10.0, 5.0, 5.0], [0.0, 0.0, 0.5, 0.5], 0.1, 0.1),
             ([7.0], [0.3], 0.1, 0.05)]
    rng = np.random.default_rng(17)
    for _ in range(300):
        L = int(rng.integers(1, 40))
        e = np.cumsum(-np.abs(rng.normal(0.0, 0.6, L))) + 12.0
        sp = np.clip(np.cumsum(np.abs(rng.normal(0.0, 0.05, L))), 0.0, 1.0)
        cases.append((e.astype(np.float32).tolist(), sp.astype(np.float32).tolist(),
                      float(np.float32(rng.uniform(0.0, 0.2))), float(np.float32(rng.uniform(0.0, 0.1)))))
    for e, sp, drop, rise in cases:
        st, got = _pivot(lib, e, sp, drop, rise)
        e32 = [float(np.float32(x)) for x in e]
        s32 = [float(np.float32(x)) for x in sp]
        assert st == 0 and got == oracle.pivot_layer(e32, s32, float(np.float32(drop)), float(np.float32(rise)))


def test_pivot_layer_rejects(lib):
    assert _pivot(lib, [], [], 0.1, 0.1)[0] == 1
    assert _pivot(lib, [1.0], [0.0], float("nan"), 0.1)[0] == 1
    assert lib.kvsel_pivot_layer(1, None, None, 0.1, 0.1, None) == 1


def test_csm_rejects(lib):
    assert lib.kvsel_csm_candidates(100, 3, 0, 0) == -1       # odd chunk
    assert lib.kvsel_csm_candidates(100, 66, 0, 0) == -1      # chunk above 64
    assert lib.kvsel_csm_candidates(100, 8, 60, 50) == -1     # sinks + recent above n
    assert lib.kvsel_csm_candidates(0, 8, 0, 0) == -1
    assert lib.kvsel_csm_candidates(100, 8, 2, 2) == 48       # 96 middle tokens: 12 chunks x 4
    assert lib.kvsel_csm_workspace_bytes(1, 100, 8, 2, 2, 49) == 0  # more merges than candidates
    need = lib.kvsel_csm_workspace_bytes(2, 100, 8, 2, 2, 10)
    assert need > 0
    # the workspace is one byte short in every call, so none can reach a launch
    ok = [2, 100, 128, 8, 2, 2, 10, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, FAKE, need - 1, None]
    assert lib.kvsel_csm(*ok) == 3  # the workspace is checked last, after every argument
    for i, bad in [(0, 0), (2, 96), (3, 5), (6, 49), (7, None), (8, None), (10, None), (11, None), (12, None),
                   (7, FAKE + 8)]:
        args = list(ok)
        args[i] = bad
        st = lib.kvsel_csm(*args)
        assert st == (2 if (i == 2) else 1), (i, bad, st)


def test_decode_rejects(lib):
    need = lib.kvsel_decode_workspace_bytes(2, 8, 2, 128, 1000)
    assert need > 0
    assert lib.kvsel_decode_workspace_bytes(2, 18, 2, 128, 1000) == 0  # 9 query heads per KV head
    assert lib.kvsel_decode_workspace_bytes(2, 8, 3, 128, 1000) == 0   # heads not a multiple
    # the workspace is one byte short in every call, so none can reach a launch
    ok = [2, 8, 2, 128, 1000, 0.0, FAKE, FAKE, FAKE, None, FAKE, FAKE, need - 1, None]
    assert lib.kvsel_decode_attention(*ok) == 3
    for i, bad, st in [(0, 0, 1), (4, 0, 1), (3, 96, 2), (1, 18, 2), (5, float("nan"), 1), (6, None, 1),
                       (7, None, 1), (8, None, 1), (10, None, 1), (7, FAKE + 8, 1)]:
        args = list(ok)
        args[i] = bad
        assert lib.kvsel_decode_attention(*args) == st, (i, bad)
