"""Token-pruned self-attention for MI355X (gfx950): a C-ABI HIP library plus a thin binding.

The compute path is libtsa.so (include/tsa.h); this package only loads it,
marshals arguments (``_binding``) and sequences the calls of one layer step
(``layer``).  Importing the package loads the library and raises if it has
not been built: there is no CPU fallback.

Docstrings label the steps as include/tsa.h does: a1 score, a2 select,
a3 compact, a4 gather, a5 QKV projection, a6 KV-cache sync, a7 attention,
a8 scatter; f1-f4 are the steps beside the layer (Euler update, pruning
mask and restoration, rotary frame-causal attention, Timeripple reuse).
"""

from . import _binding
from ._binding import (
    BF16,
    F32,
    SCORE_ABS_L1,
    SCORE_REL_L1,
    SELECT_MASK,
    SELECT_SCHEDULE,
    SELECT_THRESHOLD,
    SELECT_TOPK,
    TsaError,
    abi_version,
    assign_groups,
    attention_workspace_bytes,
    euler_update,
    frame_causal_attention,
    gather_rows,
    kv_cache_sync,
    lif_mask,
    lib,
    lib_path,
    qkv_active,
    qkv_active_rope,
    qkv_rows_to_cache,
    restore_frames,
    reuse_workspace_bytes,
    scatter_out,
    select_active,
    select_workspace_bytes,
    sparse_query_attention,
    status_string,
    reuse_noalloc_max_token_heads,
    timeripple_reuse,
    timeripple_reuse_noalloc,
    token_scores,
)
from .layer import PrunedAttentionLayer, hsa_active_count

lib()  # load now: fail loudly when the HIP library is missing

__all__ = [
    "BF16", "F32", "SCORE_ABS_L1", "SCORE_REL_L1", "SELECT_MASK", "SELECT_SCHEDULE",
    "SELECT_THRESHOLD", "SELECT_TOPK", "TsaError", "abi_version", "assign_groups", "attention_workspace_bytes", "euler_update", "frame_causal_attention", "gather_rows",
    "kv_cache_sync", "lib", "lib_path", "lif_mask", "qkv_active", "qkv_active_rope", "restore_frames", "scatter_out", "select_active",
    "select_workspace_bytes", "sparse_query_attention", "status_string", "token_scores",
    "timeripple_reuse", "timeripple_reuse_noalloc", "reuse_noalloc_max_token_heads",
    "PrunedAttentionLayer", "hsa_active_count",
]
