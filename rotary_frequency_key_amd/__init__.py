"""MI355X-native key-eviction pass of TriAttention: offset-averaged trigonometric key score,
per-unit top-B select and K/V compaction, as hand-written HIP kernels for gfx950 behind the
C interface of ``libtri.so`` (include/tri.h).

This module only marshals arguments: torch tensors -> device pointers and the current HIP
stream. Every step of the pass runs in libtri's kernels; there is no fallback. Importing it
fails when ``libtri.so`` has not been built.
"""
from ._abi import (  # noqa: F401
    TRI_BANDS_HALF_SPLIT,
    TRI_BANDS_INTERLEAVED,
    TRI_DT_BF16,
    TRI_DT_F32,
    TRI_KEYS_ROTATED,
    TRI_SELECT_HIST_FROM_SCORE,
    NOALLOC_SCRATCH_BYTES,
    InplacePlan,
    MaxPassPlan,
    PassPlan,
    ScorePlan,
    TriError,
    library_path,
    inplace_workspace_bytes,
    make_inplace_workspace,
    make_workspace,
    prune_inplace,
    prune_pass,
    prune_pass_3calls,
    prune_pass_max,
    prune_pass_noalloc,
    workspace_bytes,
    score_workspace_bytes,
    stamps_attach,
    stamps_layout,
    tri_compact_kv,
    tri_fold_weights,
    tri_score,
    tri_score_max,
    tri_select_topb,
)
