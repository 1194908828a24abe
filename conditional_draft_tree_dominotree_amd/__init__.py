"""MI355X (gfx950) conditional best-first draft-tree builder.

The compute path is the HIP library libdominotree.so (C ABI in
include/dominotree.h); `binding` marshals torch device tensors into it.
"""
from .binding import (DT_ACT_BF16, DT_BF16, DT_F32, DT_MARGINAL, DT_NORM_FULLV, DT_NORM_TOPM, DT_TIMING,
                      DT_VALIDATE, DtError, Schedule, TreeBuilder, dt_build_trees, dt_create, dt_destroy,
                      dt_draft_chain, dt_draft_chain_sample, dt_fold_state, dt_last_error, dt_phase_times,
                      dt_set_device_error, dt_set_schedule, dt_sync_status, dt_tree_attention_inputs, dt_version,
                      library_path, load_library, tree_attention_inputs)

__all__ = [
    "DT_ACT_BF16", "DT_BF16", "DT_F32", "DT_MARGINAL", "DT_NORM_FULLV", "DT_NORM_TOPM", "DT_TIMING", "DT_VALIDATE",
    "DtError", "Schedule", "TreeBuilder", "dt_build_trees", "dt_create", "dt_destroy", "dt_draft_chain",
    "dt_draft_chain_sample", "dt_fold_state", "dt_last_error", "dt_phase_times", "dt_set_device_error",
    "dt_set_schedule", "dt_sync_status", "dt_tree_attention_inputs", "dt_version", "library_path", "load_library",
    "tree_attention_inputs",
]
