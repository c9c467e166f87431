"""MI355X (gfx950) tree-masked verify/expand attention for speculative decoding.

The compute lives in ``libtreeattn.so`` (hand-written HIP kernels behind the C
ABI of ``include/tree_attn.h``); this package is its ctypes binding.  The
entry points keep the C names:

* ``tree_attn_verify``   -- tree-masked attention over every draft node
* ``tree_attn_expand``   -- the same for the w newest leaves (non-square mask)
* ``tree_attn_verify_noalloc`` -- verify with the library's fixed scratch (no allocation)
* ``tree_attn_verify_rope`` / ``tree_attn_expand_rope`` -- the same with RoPE fused in
* ``accept_greedy_path`` -- greedy longest accepted path, AL and bonus token
* ``accept_sampling_path`` -- the same by speculative sampling (temperature > 0)
* ``tree_cache_reroot``  -- evolving-tree-cache re-root with in-place KV moves
* ``tree_cache_reroot_draft`` -- the same, moving the draft's tokens and re-based scores too
* ``tree_accept_reroot`` -- ``accept_greedy_path`` + ``tree_cache_reroot`` in two launches
* ``tree_expand_top_w``  -- maximum-likelihood expansion: append the w best leaves
* ``tree_rope_append``   -- RoPE at tree positions + KV append of the new nodes
* ``tree_token_walk``    -- draft side: walk along the verified tokens (re-root path)
* ``tree_select_subtree``-- draft side: the size-bs subtree to send
"""
from ._lib import (  # noqa: F401
    EXPORTED_SYMBOLS,
    KVCache,
    TA_BF16,
    TA_F32,
    TA_MAX_NODES,
    TreeAttnError,
    Workspace,
    accept_greedy_path,
    accept_sampling_path,
    accept_sampling_workspace_bytes,
    load_library,
    ta_last_error,
    ta_status_string,
    ta_version,
    tree_attn_expand,
    tree_attn_verify,
    tree_attn_verify_noalloc,
    tree_attn_verify_rope,
    tree_attn_expand_rope,
    tree_attn_workspace_bytes,
    tree_cache_reroot,
    tree_cache_reroot_draft,
    tree_accept_reroot,
    tree_accept_reroot_workspace_bytes,
    tree_expand_top_w,
    tree_expand_top_w_workspace_bytes,
    tree_rope_append,
    tree_select_subtree,
    tree_token_walk,
)

__version__ = "0.1.0"
