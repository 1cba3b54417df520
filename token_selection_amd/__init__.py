"""kvsel: attention-saliency KV token selection for MI355X (gfx950).

The work runs in ``libkvsel.so`` (hand-written HIP kernels behind the C ABI
of ``include/kvsel.h``); ``token_selection_amd.kvsel`` is its ctypes binding.
"""

from .kvsel import (  # noqa: F401
    KVSEL_ACC_ADD,
    KVSEL_ACC_HEAD_MEAN,
    KvselError,
    budget_from_rate,
    kvsel_accumulate,
    kvsel_gather,
    kvsel_score,
    kvsel_score_workspace_bytes,
    kvsel_topk,
    kvsel_topk_workspace_bytes,
    library_path,
    load_library,
    score_desc,
    status_string,
    version,
)
