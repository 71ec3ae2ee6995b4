"""MI355X-native sparse-embedding + dot-interaction core of a DLRM-style recommender.

The compute lives in ``libembcore.so`` (HIP kernels for gfx950 behind the C ABI in
``include/embcore.h``); ``embcore`` is its Python binding and ``synth`` makes seeded
synthetic inputs shaped like the workloads of the page "DLRM For PyTorch".
"""
from .embcore import (  # noqa: F401
    Bags,
    EmbcoreError,
    Tables,
    alloc_workspace,
    cat_interact_bwd,
    cat_interact_fwd,
    dot_interact_bwd,
    dot_interact_fwd,
    el_last_error,
    el_validate_bags,
    el_version,
    hbm_calib,
    emb_bag_fwd,
    emb_cat_fwd,
    emb_dot_bwd,
    emb_dot_fwd,
    emb_grad_apply,
    emb_grad_prepare,
    emb_grad_reduce_update,
    emb_grad_reduce_update_noalloc,
    emb_grad_sort,
    emb_grad_workspace_bytes,
    bce_logits,
    bce_workspace_bytes,
    linear_bwd,
    linear_bwd_workspace_bytes,
    linear_fwd,
    relu_bwd,
    sgd_dense,
)
