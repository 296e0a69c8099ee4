"""libspecverify: batched draft verification for speculative decoding on
MI355X (gfx950), as hand-written HIP kernels behind a C ABI.

The Python surface is a thin ctypes binding (``_binding``); every step of
the computation runs in the HIP library.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MAX_GAMMA,
    MAX_TREE_NODES,
    MODE_GREEDY,
    MODE_LMHEAD,
    MODE_ROWSTATS,
    MODE_SAMPLE,
    MODE_TREE,
    MODE_TREE_EXPAND,
    MODE_TREE_SAMPLE,
    SPEC_BF16,
    SPEC_F32,
    SpecError,
    W_DV,
    W_VD,
    kv_compact,
    lib,
    lmhead_logits_view,
    lmhead_project,
    lmhead_verify,
    new_tree_table,
    new_workspace,
    PARTIAL_DTYPE,
    probe_probs,
    row_partials,
    row_stats,
    tree_build,
    tree_expand,
    verify_greedy,
    verify_sample,
    verify_tree,
    verify_tree_sample,
    workspace_bytes,
)
