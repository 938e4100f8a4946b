"""MI355X-native DLRMv1 forward hot path.

The compute lives in libdlrm_mi355x.so (hand-written HIP kernels for gfx950
behind the C ABI of include/dlrm_embedding_bag.h).  `abi` is the ctypes
binding with the same entry-point names; `inputs` draws seeded synthetic
inputs.  Importing this package loads nothing; the library is loaded on the
first call and a missing library raises.
"""
from .abi import (  # noqa: F401
    DlrmError, DlrmModel, DlrmPlan, dlrm_emb_interact, dlrm_emb_interact_dots, dlrm_emb_interact_pool, dlrm_forward,
    dlrm_forward_workspace_bytes, dlrm_interact_lower_tri, emb_bag_pool, emb_bag_sum_multi,
    linear_bias_act, linear_bias_act_split, load, mlp_forward)
