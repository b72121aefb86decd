"""MI355X-native branch-parallel target scoring for SpecOPD.

The computation lives in libspecopd.so (HIP kernels for gfx950 behind the C
ABI of include/specopd.h); this package is its thin Python binding.
"""

from ._lib import (  # noqa: F401
    EXPORTS, LIB, LIB_PATH, SpecopdError, TreeAttnDesc, E2etvDesc, SPECOPD_OK,
    SPECOPD_ERR_INVALID_ARGUMENT, SPECOPD_ERR_UNSUPPORTED, SPECOPD_ERR_WORKSPACE, SPECOPD_ERR_HIP,
    SPECOPD_ERR_DEVICE_VALIDATION, SPECOPD_F32, SPECOPD_BF16, SPECOPD_TREE_BATCH_INVARIANT, SPECOPD_E2ETV_DEFER_ALL, status_string, specopd_version,
    tree_attn_desc, e2etv_desc, specopd_tree_attn_workspace_size, specopd_tree_attn_fwd,
    specopd_tree_attn_device_status, specopd_e2etv_workspace_size, specopd_e2etv_fwd_bwd,
    specopd_e2etv_device_status, specopd_e2etv_fwd_bwd_noalloc, E2ETV_NOALLOC_SCRATCH_BYTES,
    specopd_kernel_timing, specopd_kernel_time, workspace, tree_attn, specopd_score_rows, score_rows,
    e2etv, PrefillDesc, prefill_desc, specopd_prefill_workspace_size, specopd_prefill_fwd, prefill,
    GdnDesc, gdn_desc, specopd_gdn_workspace_size, specopd_gdn_replay_fwd, specopd_gdn_device_status,
    gdn_replay, GdnConvDesc, gdn_conv_desc, specopd_gdn_conv_fwd, gdn_conv, SPECOPD_GDN_CONV_L2NORM,
    QsaDesc, qsa_desc, specopd_qsa_trunk_groups_fwd, specopd_qsa_workspace_size, specopd_qsa_select_fwd,
    specopd_qsa_device_status, qsa_trunk_groups, qsa_select,
    LmHeadDesc, lmhead_desc, specopd_lmhead_e2etv_workspace_size, specopd_lmhead_e2etv_fwd_bwd,
    specopd_lmhead_e2etv_device_status, lmhead_e2etv,
)
